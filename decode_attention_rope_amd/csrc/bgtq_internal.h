// Internal declarations shared by the host API and the kernel translation unit.
#pragma once

#include <cstddef>
#include <cstdint>

#include <hip/hip_runtime.h>

#include "bgtq.h"

namespace bgtq {

constexpr int kMaxBits = 8;
constexpr int kMaxGroups = 8;        // widths 1..8 -> at most 8 width groups
constexpr int kTile = 64;            // token slots per cache tile
constexpr int kEnergyChunk = 256;    // tokens per fixed-order energy partial sum
constexpr int kQPad = 16;            // query-head padding of the rotated-query workspace

// Per-(sequence, KV head) description of the width groups and the K record, written by
// the allocation kernel.  Storage position p holds original coordinate perm[p], belongs
// to width group group[p] and starts at record bit offset[p].
struct alignas(16) HeadLayout {
  int32_t n_groups;                 // g_K, number of width groups (widths >= 1)
  int32_t d_eff;                    // coded coordinates (blocks of width >= 1, two each)
  int32_t code_bits;                // 2 * sum of block widths
  int32_t chunks;                   // 16-byte chunks per K record
  int32_t g_width[kMaxGroups];      // descending
  int32_t g_first[kMaxGroups];      // first storage position
  int32_t g_m[kMaxGroups];          // coordinates in the group
  int32_t g_bitoff[kMaxGroups];     // record bit offset of the group's first code
  uint8_t perm[BGTQ_MAX_HEAD_DIM];
  uint8_t group[BGTQ_MAX_HEAD_DIM];
  uint16_t offset[BGTQ_MAX_HEAD_DIM];
  uint8_t reserved[BGTQ_LAYOUT_BYTES - 16 - 4 * 4 * kMaxGroups - 4 * BGTQ_MAX_HEAD_DIM];
};
static_assert(sizeof(HeadLayout) == BGTQ_LAYOUT_BYTES, "layout descriptor size");

// Frozen quantizer tables (fp32 as the kernels read them; fp64 distortions).
struct Tables {
  float thr[kMaxBits][255];   // thr[b-1][k], k < 2^b - 1, ascending
  float cen[kMaxBits][256];   // cen[b-1][k], k < 2^b, ascending
  double dgain[kMaxBits];     // dist[b] - dist[b+1], b = 0..7
  double dist[kMaxBits + 1];  // fl32(D(b)), dist[0] = 1
};

const Tables& host_tables();

inline int record_chunks(int k_width_sum) { return (2 * k_width_sum + 127) / 128; }
inline size_t rot_bank_offset(int m) {  // floats before the m x m matrix (m even)
  size_t o = 0;
  for (int k = 2; k < m; k += 2) o += size_t(k) * k;
  return o;
}
int decode_splits(int batch, int n_kv_heads, int64_t capacity);

// ---------------------------------------------------------------- launchers (kernels.hip)
hipError_t upload_tables(const Tables& t);

hipError_t launch_energy(const void* keys, bgtq_dtype dt, int n_heads, int64_t n_tokens, int d,
                         int64_t sh, int64_t st, int pairing, double* energy, double* partial,
                         hipStream_t s);

hipError_t launch_allocate(const double* energy, int n_heads, int n_blocks, int increments, int b_min,
                           int b_max, int pairing, uint8_t* widths, HeadLayout* layouts, hipStream_t s);

struct AppendArgs {
  const float* rot_bank;
  const float* rot_v;
  const void* keys;
  const void* values;
  int64_t stride_seq, stride_head, stride_token;
  uint8_t* k_codes;
  uint16_t* k_norms;
  uint8_t* v_codes;
  uint16_t* v_norms;
  int32_t* lengths;
  const HeadLayout* layouts;
  int32_t* status;
  int64_t capacity;
  int64_t n_new;
  int seq_begin;
  int n_kv_heads;
  int d;
  int v_bits;
  int chunks;
};
hipError_t launch_append(const AppendArgs& a, bgtq_dtype dt, int n_seqs, hipStream_t s);

struct DecodeArgs {
  const float* rot_bank;
  const float* rot_v;
  const void* q;
  const int64_t* q_pos;
  const uint8_t* k_codes;
  const uint16_t* k_norms;
  const uint8_t* v_codes;
  const uint16_t* v_norms;
  const int32_t* lengths;
  const HeadLayout* layouts;
  float* out;
  float* logits;
  float* qrot;        // [batch][n_kv][d][kQPad]
  float* partial;     // [batch][n_q][n_split][d + 2]
  double rope_theta;
  float scale;
  int64_t capacity;
  int batch, n_q, n_kv, group, d, v_bits, chunks, n_split, pairing;
};
hipError_t launch_decode(const DecodeArgs& a, bgtq_dtype q_dt, hipStream_t s);

}  // namespace bgtq
