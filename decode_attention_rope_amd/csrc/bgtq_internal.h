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
constexpr int kMaxKSteps = BGTQ_MAX_HEAD_DIM / 32 + 10;  // 32-position MFMA k-steps per head
constexpr int kSegLen = 8;
constexpr int kMaxRecordDwords = 2 * BGTQ_MAX_BITS * BGTQ_MAX_HEAD_DIM / 2 / 32;   // 64           // storage positions per MFMA k-segment (one lane's share of a k-step)

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
  // Matrix-core view of the K record.  Every width group is cut into segments of at most 8
  // storage positions, taken in storage order; k-step s holds segments 4 s + j (lane group j)
  // from at most two groups: group kgroups[s] & 0xff feeds output columns 0-7 and group
  // kgroups[s] >> 8 columns 8-15, so every group's partial logit can be scaled by its own
  // fp32 norm.  seg = bit offset | width << 16 | group << 20 | count << 24 | half << 28;
  // an unused slot decodes bit 0 with width 1 and meets zero query entries.
  int32_t n_ksteps;
  int32_t reserved0[3];
  uint32_t seg[4 * kMaxKSteps];
  uint32_t kgroups[kMaxKSteps];
  uint16_t kpos[BGTQ_MAX_HEAD_DIM];   // storage position -> k index (32 s + 8 j + e)
  // record dword w holds bits of storage positions dw_first[w] .. dw_end[w] - 1
  uint16_t dw_first[kMaxRecordDwords];
  uint16_t dw_end[kMaxRecordDwords];
  uint8_t reserved[BGTQ_LAYOUT_BYTES - 16 - 4 * 4 * kMaxGroups - 4 * BGTQ_MAX_HEAD_DIM - 16 -
                   20 * kMaxKSteps - 2 * BGTQ_MAX_HEAD_DIM - 4 * kMaxRecordDwords];
};
static_assert(sizeof(HeadLayout) == BGTQ_LAYOUT_BYTES, "layout descriptor size");
static_assert(offsetof(HeadLayout, seg) % 16 == 0, "a k-step's four segments are read as one 16-byte word");

// Frozen quantizer tables (fp32 as the kernels read them; fp64 distortions).
constexpr int kPairWords = 1364;    // fp16 pair tables of widths 1..5: sum over w of 4^w entries
constexpr int kSingleHalves = 510;  // fp16 level tables of widths 1..8 (width w at 2^w - 2)

struct Tables {
  float thr[kMaxBits][255];   // thr[b-1][k], k < 2^b - 1, ascending
  float cen[kMaxBits][256];   // cen[b-1][k], k < 2^b, ascending
  // decoder tables: fp16 (nearest-even) of cen.  pair[(4^w - 4)/3 + (c0 | c1 << w)] holds the
  // levels of codes c0 (low half) and c1 (high half) of width w <= 5; single[] widths 1..8.
  uint32_t pair[kPairWords];
  uint16_t single[kSingleHalves];
  // the same levels split as hi + lo, hi = fp16(cen), lo = fp16(cen - hi): hi + lo carries the
  // fp32 centroid to about 2^-22 relative.  pair_hl[i] = (pair hi halves, pair lo halves);
  // single_hl[] = hi | lo << 16, widths 1..8 at 2^w - 2.
  uint32_t pair_hl[kPairWords][2];
  uint32_t single_hl[kSingleHalves];
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
int decode_splits(int batch, int n_kv_heads, int64_t capacity, bool mfma);
// the streamed matrix-core split pass: whether it serves a cache geometry (head dims 64/128,
// tiles that fit its staging), and its split count per (sequence, KV head)
bool decode_stream_fits(int d, int chunks, int v_bits);
int decode_stream_splits(int batch, int n_kv_heads);
// whether its remaining tiles go out whole (a launch of several rounds of workgroups) rather than
// as quarter units
bool decode_stream_whole_tiles(int batch, int n_kv_heads);
// splits that attend over a window of w tokens (at most two 64-token tiles each)
inline int window_splits(int w) { return w > 0 ? ((w + kTile - 1) / kTile + 2) / 2 : 0; }
constexpr int kMaxWindowSplits = (BGTQ_MAX_WINDOW / kTile + 2) / 2;
size_t decode_qrot_bytes(int batch, int n_kv_heads, int d);

// ---------------------------------------------------------------- launchers (kernels.hip)
hipError_t upload_tables(const Tables& t);

hipError_t launch_energy(const void* keys, bgtq_dtype dt, int n_heads, int64_t n_tokens, int d,
                         int64_t sh, int64_t st, int pairing, double* energy, double* partial,
                         hipStream_t s);

// prefill of one sequence's heads: energy partials, then the final sums and the allocation
// in one kernel (per-head widths and layouts written at `widths`, `layouts`)
hipError_t launch_prefill_alloc(const void* keys, bgtq_dtype dt, int n_heads, int64_t n_tokens, int d, int64_t sh,
                               int64_t st, int pairing, double* partial, int increments, int b_min, int b_max,
                               double* energy_out, uint8_t* widths, HeadLayout* layouts, hipStream_t s);

hipError_t launch_allocate(const double* energy, int n_heads, int n_blocks, int increments, int b_min,
                           int b_max, int pairing, uint8_t* widths, HeadLayout* layouts, hipStream_t s);

struct AppendArgs {
  const float* rot_bank;
  const float* rot_v;
  const float* rot_bank_t;
  const float* rot_v_t;
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
  int advance;        // lengths[] advanced after the append (a decode step leaves that to the merge)
  uint16_t* k_window; // fp16 recent keys [batch][n_kv][window][d], token t at slot t % window
  int window;         // 0: no window
  const uint4* givens;  // structured rotations (header, then records), or null for dense ones
  int kv_bf16;        // keys and values are bf16 (the decode step's append role)
};
hipError_t launch_append(const AppendArgs& a, bgtq_dtype dt, int n_seqs, hipStream_t s);

struct DecodeArgs {
  const float* rot_bank;
  const float* rot_v;
  const float* rot_bank_t;
  const void* q;
  const int64_t* q_pos;
  const uint8_t* k_codes;
  const uint16_t* k_norms;
  const uint8_t* v_codes;
  const uint16_t* v_norms;
  int32_t* lengths;
  const HeadLayout* layouts;
  float* out;
  float* logits;
  float* qrot;        // [batch][n_kv][d][kQPad] fp32 (vector-ALU kernel)
  float* partial;     // [batch][n_q][n_split][d] split accumulators
  float2* part_ml;    // [batch][n_q][n_split] split (running max, row sum)
  int32_t* step_flag; // [batch][n_kv] decode step: new length once the append role's stores are released
  int step_spin;      // decode step: bound of the wait for the append role (spins of a few hundred cycles)
  double rope_theta;
  double inv_freq[BGTQ_MAX_HEAD_DIM / 2];   // rope_theta^(-2j/d), fp64, computed on the host
  float scale;
  int64_t capacity;
  int batch, n_q, n_kv, group, d, v_bits, chunks, n_split, pairing;
  int step;           // decode step: one token is appended beside the pass (its append role)
  int use_mfma;
  int use_stream;             // the streamed matrix-core split pass (no window, head dims 64/128)
  int stream_whole_tiles;     // streamed pass: remaining tiles go out whole (else as quarter units)
  const uint16_t* k_window;   // fp16 recent keys (see AppendArgs)
  int window;                 // 0: no window
  int n_wsplit;               // the first n_wsplit splits attend over the window's tokens
  const uint4* givens;        // structured rotations (see AppendArgs), or null for dense ones
};
hipError_t launch_decode(const DecodeArgs& a, bgtq_dtype q_dt, hipStream_t s);
// decode step on the matrix-core path: append one token per sequence and attend (da.step = 1,
// da.step_flag set, aa.advance = 0)
hipError_t launch_decode_step(const AppendArgs& aa, const DecodeArgs& da, bgtq_dtype kv_dt, bgtq_dtype q_dt,
                              hipStream_t s);
// the decode step's flags: one int per (sequence, KV head), zero between steps
size_t decode_step_bytes(int batch, int n_kv_heads);
// clears n step flags with a fill kernel (no memset node, so the call can be captured)
hipError_t launch_clear_flags(int32_t* flags, int n, hipStream_t s);
// device address of the current device's allocation-free scratch (BGTQ_NOALLOC_SCRATCH_BYTES)
hipError_t scratch_address(void** ptr);

// key-only logit error (diagnostic.hip)
constexpr int kErrChunk = 256;       // tokens per workgroup and per partial sum
struct LogitErrArgs {
  const void* q;
  const int64_t* q_pos;
  const void* keys;
  int64_t stride_seq, stride_head, stride_token;
  const int32_t* lengths;
  const float* logits;
  double* partial;    // [batch][n_q][n_chunk] per-chunk sums of |error|
  double* mae;        // [batch][n_q]
  double rope_theta;
  double inv_freq[BGTQ_MAX_HEAD_DIM / 2];
  float scale;
  int64_t capacity;
  int batch, n_q, n_kv, group, d, pairing, n_chunk;
};
hipError_t launch_logit_error(const LogitErrArgs& a, bgtq_dtype k_dt, bgtq_dtype q_dt, hipStream_t s);

hipError_t launch_transpose_rotations(const float* rot_bank, const float* rot_v, int d, float* rot_bank_t,
                                      float* rot_v_t, hipStream_t s);

}  // namespace bgtq
