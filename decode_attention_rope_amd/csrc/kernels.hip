// HIP kernels of the Block-GTQ packed-cache decode path, written for gfx950 (CDNA4, wave64).
//
// Method: "RoPE-Aware Bit Allocation for KV-Cache Quantization" (arXiv 2606.24033), abstract.
// Each kernel states the reading of the abstract it implements.  Kernels that must agree
// bit for bit with the reference arithmetic (energy, allocation, quantize-and-pack) are
// compiled without floating-point contraction (-ffp-contract=off) and use only correctly
// rounded fp32/fp64 operations in a fixed order; decode attention uses explicit fmaf.

#include <hip/hip_runtime.h>

#include "bgtq_internal.h"

namespace bgtq {
namespace {

typedef const float __attribute__((address_space(4))) cfloat;
typedef const HeadLayout __attribute__((address_space(4))) cLayout;

__constant__ float c_thr[kMaxBits][255];
__constant__ float c_cen[kMaxBits][256];
__constant__ double c_dgain[kMaxBits];

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr double kTwoPi = 6.283185307179586476925286766559;

__device__ __forceinline__ float load_f(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float load_f(const uint16_t* p, int64_t i) {
  return __uint_as_float(uint32_t(p[i]) << 16);  // bf16 -> fp32 is exact
}
__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) {
  const _Float16 h = (_Float16)x;  // round to nearest even
  return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ float f16_bits_to_f32(uint16_t u) {
  return (float)__builtin_bit_cast(_Float16, u);
}

// Orders LDS traffic between lanes of one wavefront (all lanes run in lockstep).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Number of sorted thresholds strictly below z (the b-bit code of z).
__device__ __forceinline__ int code_of(const float* thr, int bits, float z) {
  int code = 0;
  for (int b = bits - 1; b >= 0; --b) {
    const int cand = code | (1 << b);
    if (z > thr[cand - 1]) code = cand;
  }
  return code;
}

__device__ __forceinline__ size_t bank_offset(int m) {  // sum of k*k for even k < m
  const size_t h = size_t(m) / 2 - 1;                   // number of smaller sizes
  return 4 * (h * (h + 1) * (2 * h + 1) / 6);
}

// ===================================================================== block energy
// Label-free energy of RoPE block j (abstract: one score per RoPE block, per layer and KV
// head, no labels needed).  Reading: mean over tokens of the squared norm of the block's
// two coordinates, fp64, summed in ascending t within 256-token chunks, chunks in
// ascending order.  Pass 1: one thread per (head, chunk, block); lanes run over blocks
// so every token row is read coalesced.  Pass 2: one thread per (head, block).
template <typename T>
__global__ void k_energy_partial(const T* __restrict__ keys, int n_heads, int64_t n_tokens, int n,
                                 int64_t sh, int64_t st, int pairing, int n_chunks,
                                 double* __restrict__ part) {
  const int64_t gid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (gid >= int64_t(n_heads) * n_chunks * n) return;
  const int j = int(gid % n);
  const int64_t rest = gid / n;
  const int c = int(rest % n_chunks);
  const int h = int(rest / n_chunks);
  const int ca = pairing ? 2 * j : j, cb = pairing ? 2 * j + 1 : j + n;
  const T* base = keys + int64_t(h) * sh;
  const int64_t t0 = int64_t(c) * kEnergyChunk;
  const int64_t t1 = t0 + kEnergyChunk < n_tokens ? t0 + kEnergyChunk : n_tokens;
  double acc = 0.0;
  for (int64_t t = t0; t < t1; ++t) {
    const double x0 = (double)load_f(base, t * st + ca);
    const double x1 = (double)load_f(base, t * st + cb);
    const double e = x0 * x0 + x1 * x1;
    acc = acc + e;
  }
  part[(int64_t(h) * n_chunks + c) * n + j] = acc;
}

__global__ void k_energy_final(const double* __restrict__ part, int n_heads, int n_chunks, int n,
                               int64_t n_tokens, double* __restrict__ out) {
  const int gid = blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= n_heads * n) return;
  const int h = gid / n, j = gid % n;
  double tot = 0.0;
  for (int c = 0; c < n_chunks; ++c) tot = tot + part[(int64_t(h) * n_chunks + c) * n + j];
  out[gid] = tot / (double)n_tokens;
}

// ===================================================================== greedy allocation
// Integer widths by marginal gain (abstract: greedy, integer widths, more bits where the
// energy is high, matched budget).  Reading: every block starts at b_min; each of the
// `increments` steps gives one bit to the block of largest fp64 gain E_j*(D(b_j)-D(b_j+1))
// among blocks below b_max, ties to the lowest j.  One wavefront per head, block j on
// lane j % 64; the arg-max runs over the wave with a (gain, -j) order.  Lane 0 then
// derives the width groups and the K record layout.
__global__ __launch_bounds__(64) void k_allocate(const double* __restrict__ energy, int n, int increments,
                                                 int b_min, int b_max, int pairing,
                                                 uint8_t* __restrict__ widths,
                                                 HeadLayout* __restrict__ layouts) {
  __shared__ int w_s[128];
  __shared__ HeadLayout lay;
  const int h = blockIdx.x, lane = threadIdx.x;
  const int j0 = lane, j1 = lane + 64;
  const double e0 = j0 < n ? energy[int64_t(h) * n + j0] : 0.0;
  const double e1 = j1 < n ? energy[int64_t(h) * n + j1] : 0.0;
  int w0 = b_min, w1 = b_min;
  for (int it = 0; it < increments; ++it) {
    const double g0 = (j0 < n && w0 < b_max) ? e0 * c_dgain[w0] : -1.0;
    const double g1 = (j1 < n && w1 < b_max) ? e1 * c_dgain[w1] : -1.0;
    double g = g0;
    int j = j0;
    if (g1 > g0) { g = g1; j = j1; }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const double go = __shfl_xor(g, off);
      const int jo = __shfl_xor(j, off);
      if (go > g || (go == g && jo < j)) { g = go; j = jo; }
    }
    if (j == j0) ++w0;
    else if (j == j1) ++w1;
  }
  if (j0 < n) { w_s[j0] = w0; widths[int64_t(h) * n + j0] = uint8_t(w0); }
  if (j1 < n) { w_s[j1] = w1; widths[int64_t(h) * n + j1] = uint8_t(w1); }
  uint32_t* lw = reinterpret_cast<uint32_t*>(&lay);
  for (int i = lane; i < int(sizeof(HeadLayout) / 4); i += 64) lw[i] = 0;
  __syncthreads();
  if (lane == 0) {
    int pos = 0, bit = 0, g = 0;
    for (int w = kMaxBits; w >= 1; --w) {
      const int first = pos, bit0 = bit;
      for (int jj = 0; jj < n; ++jj) {
        if (w_s[jj] != w) continue;
        const int ca = pairing ? 2 * jj : jj, cb = pairing ? 2 * jj + 1 : jj + n;
        lay.perm[pos] = uint8_t(ca); lay.group[pos] = uint8_t(g); lay.offset[pos] = uint16_t(bit);
        bit += w; ++pos;
        lay.perm[pos] = uint8_t(cb); lay.group[pos] = uint8_t(g); lay.offset[pos] = uint16_t(bit);
        bit += w; ++pos;
      }
      if (pos > first) {
        lay.g_width[g] = w; lay.g_first[g] = first; lay.g_m[g] = pos - first; lay.g_bitoff[g] = bit0;
        ++g;
      }
    }
    lay.n_groups = g; lay.d_eff = pos; lay.code_bits = bit; lay.chunks = (bit + 127) / 128;
  }
  __syncthreads();
  uint32_t* dst = reinterpret_cast<uint32_t*>(layouts + h);
  for (int i = lane; i < int(sizeof(HeadLayout) / 4); i += 64) dst[i] = lw[i];
}

// ===================================================================== quantize + append
// TQ-MSE quantize-and-pack of new tokens (abstract: Block-GTQ is built on TurboQuant-MSE;
// keys at the allocated per-block widths, values at one width; packed cache).  Reading:
// width groups are TQ-MSE vectors: fp32 norm (sequential sum of squares, sqrt), y = R x
// (sequential dot products, no fused multiply-add), z = (y / n) * fl32(sqrt(m)), code =
// number of fp32 thresholds below z, norm stored as fp16.  One workgroup owns 32 slots
// (half a tile) of one (sequence, KV head); half tiles never share a packed dword, so no
// atomics are needed.  Slots that are not being appended keep their bits.
constexpr int kHalf = 32;

template <typename T>
__global__ __launch_bounds__(256) void k_append(AppendArgs a) {
  extern __shared__ float sm[];
  const int d = a.d, n = d / 2;
  const int si = blockIdx.z, s = a.seq_begin + si, hk = blockIdx.y;
  const int tid = threadIdx.x, nt = blockDim.x;
  const int64_t len = a.lengths[s];
  if (len + a.n_new > a.capacity) {
    if (blockIdx.x == 0 && hk == 0 && tid == 0 && a.status) atomicOr(a.status, 1);
    return;
  }
  const int64_t ht = len / kHalf + blockIdx.x;
  const int64_t lo = len > ht * kHalf ? len : ht * kHalf;
  const int64_t hi = (len + a.n_new) < (ht + 1) * kHalf ? (len + a.n_new) : (ht + 1) * kHalf;
  if (lo >= hi) return;
  const int64_t tile = ht / 2;
  const int half = int(ht & 1);
  const int XS = d + 1;
  float* xs = sm;                                   // [32][d+1]
  float* thr = xs + kHalf * XS;                     // [8][255]
  float* knrm = thr + kMaxBits * 255;               // [32][8]
  float* vnrm = knrm + kHalf * kMaxGroups;          // [32]
  uint8_t* kcode = reinterpret_cast<uint8_t*>(vnrm + kHalf);   // [32][256]
  uint8_t* vcode = kcode + kHalf * BGTQ_MAX_HEAD_DIM;            // [32][256]
  int* pb = reinterpret_cast<int*>(vcode + kHalf * BGTQ_MAX_HEAD_DIM);  // [64] first position per dword
  int* pe = pb + 64;                                                    // [64] end position per dword

  const HeadLayout& L = a.layouts[int64_t(s) * a.n_kv_heads + hk];
  const int ng = L.n_groups, d_eff = L.d_eff, n_dw = 4 * a.chunks;
  const size_t reg = size_t(s) * a.n_kv_heads + hk;
  const int64_t tiles = a.capacity / kTile;
  (void)n;

  for (int i = tid; i < kMaxBits * 255; i += nt) thr[i] = c_thr[i / 255][i % 255];
  for (int w = tid; w < n_dw; w += nt) {
    int p = 0;
    while (p < d_eff && int(L.offset[p]) + L.g_width[L.group[p]] <= 32 * w) ++p;
    int q = p;
    while (q < d_eff && int(L.offset[q]) < 32 * w + 32) ++q;
    pb[w] = p; pe[w] = q;
  }
  const T* kin = static_cast<const T*>(a.keys) + si * a.stride_seq + hk * a.stride_head;
  const T* vin = static_cast<const T*>(a.values) + si * a.stride_seq + hk * a.stride_head;
  for (int idx = tid; idx < kHalf * d; idx += nt) {
    const int r = idx / d, c = idx % d;
    const int64_t slot = ht * kHalf + r;
    xs[r * XS + c] = (slot >= lo && slot < hi) ? load_f(kin, (slot - len) * a.stride_token + c) : 0.0f;
  }
  __syncthreads();
  // key group norms
  for (int it = tid; it < kHalf * ng; it += nt) {
    const int r = it % kHalf, g = it / kHalf;
    const int first = L.g_first[g], m = L.g_m[g];
    float ss = 0.0f;
    for (int k = 0; k < m; ++k) {
      const float v = xs[r * XS + L.perm[first + k]];
      ss = ss + v * v;
    }
    knrm[r * kMaxGroups + g] = sqrtf(ss);
  }
  __syncthreads();
  // key codes, storage order
  for (int it = tid; it < kHalf * d_eff; it += nt) {
    const int r = it % kHalf, p = it / kHalf;
    const int g = L.group[p], w = L.g_width[g], m = L.g_m[g], first = L.g_first[g];
    const float* R = a.rot_bank + bank_offset(m) + size_t(p - first) * m;
    float acc = 0.0f;
    for (int k = 0; k < m; ++k) acc = acc + R[k] * xs[r * XS + L.perm[first + k]];
    const float nv = knrm[r * kMaxGroups + g];
    int code = 0;
    if (nv != 0.0f) {
      const float z = (acc / nv) * sqrtf(float(m));
      code = code_of(thr + (w - 1) * 255, w, z);
    }
    kcode[r * BGTQ_MAX_HEAD_DIM + p] = uint8_t(code);
  }
  __syncthreads();
  for (int idx = tid; idx < kHalf * d; idx += nt) {
    const int r = idx / d, c = idx % d;
    const int64_t slot = ht * kHalf + r;
    xs[r * XS + c] = (slot >= lo && slot < hi) ? load_f(vin, (slot - len) * a.stride_token + c) : 0.0f;
  }
  __syncthreads();
  for (int r = tid; r < kHalf; r += nt) {
    float ss = 0.0f;
    for (int k = 0; k < d; ++k) {
      const float v = xs[r * XS + k];
      ss = ss + v * v;
    }
    vnrm[r] = sqrtf(ss);
  }
  __syncthreads();
  const float sd = sqrtf(float(d));
  for (int it = tid; it < kHalf * d; it += nt) {
    const int r = it % kHalf, i = it / kHalf;
    const float* R = a.rot_v + size_t(i) * d;
    float acc = 0.0f;
    for (int k = 0; k < d; ++k) acc = acc + R[k] * xs[r * XS + k];
    const float nv = vnrm[r];
    int code = 0;
    if (nv != 0.0f) code = code_of(thr + (a.v_bits - 1) * 255, a.v_bits, (acc / nv) * sd);
    vcode[r * BGTQ_MAX_HEAD_DIM + i] = uint8_t(code);
  }
  __syncthreads();
  // pack key records (one thread per (slot, record dword))
  uint32_t* kc = reinterpret_cast<uint32_t*>(a.k_codes) + reg * tiles * a.chunks * kTile * 4;
  for (int it = tid; it < kHalf * n_dw; it += nt) {
    const int r = it % kHalf, w = it / kHalf;
    const int64_t slot = ht * kHalf + r;
    if (slot < lo || slot >= hi) continue;
    uint32_t v = 0;
    for (int p = pb[w]; p < pe[w]; ++p) {
      const uint32_t c = kcode[r * BGTQ_MAX_HEAD_DIM + p];
      const int o = int(L.offset[p]) - 32 * w;
      v |= o >= 0 ? (c << o) : (c >> (-o));
    }
    kc[((tile * a.chunks + w / 4) * kTile + (slot % kTile)) * 4 + (w % 4)] = v;
  }
  // pack value segments (one thread per (coordinate, segment dword) of this half tile)
  const int bv = a.v_bits;
  uint32_t* vc = reinterpret_cast<uint32_t*>(a.v_codes) + reg * tiles * d * 2 * bv;
  const uint32_t vmask = (1u << bv) - 1u;
  for (int it = tid; it < d * bv; it += nt) {
    const int i = it / bv, w = half * bv + it % bv;
    uint32_t* addr = vc + (size_t(tile) * d + i) * 2 * bv + w;
    uint32_t v = *addr;
    const int bit0 = 32 * w;
    for (int j = bit0 / bv; j * bv < bit0 + 32; ++j) {
      const int64_t slot = tile * kTile + j;
      if (slot < lo || slot >= hi) continue;
      const uint32_t c = vcode[int(slot - ht * kHalf) * BGTQ_MAX_HEAD_DIM + i];
      const int o = j * bv - bit0;
      if (o >= 0) v = (v & ~(vmask << o)) | (c << o);
      else v = (v & ~(vmask >> (-o))) | (c >> (-o));
    }
    *addr = v;
  }
  // norms
  uint16_t* kn = a.k_norms + reg * tiles * kMaxGroups * kTile;
  uint16_t* vn = a.v_norms + reg * tiles * kTile;
  for (int it = tid; it < kHalf * ng; it += nt) {
    const int r = it % kHalf, g = it / kHalf;
    const int64_t slot = ht * kHalf + r;
    if (slot < lo || slot >= hi) continue;
    kn[(tile * kMaxGroups + g) * kTile + slot % kTile] = f32_to_f16_bits(fminf(knrm[r * kMaxGroups + g], 65504.0f));
  }
  for (int r = tid; r < kHalf; r += nt) {
    const int64_t slot = ht * kHalf + r;
    if (slot < lo || slot >= hi) continue;
    vn[tile * kTile + slot % kTile] = f32_to_f16_bits(fminf(vnrm[r], 65504.0f));
  }
}

__global__ void k_advance(int32_t* __restrict__ lengths, int seq_begin, int n_seqs, int64_t n_new,
                          int64_t capacity) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n_seqs) return;
  const int s = seq_begin + i;
  if (lengths[s] + n_new <= capacity) lengths[s] = int32_t(lengths[s] + n_new);
}

// ===================================================================== decode attention
// RoPE query-key logits over the packed cache (abstract: the logit is a sum over 2-D RoPE
// blocks; the serving path attends over the packed cache).  The key reconstruction of
// width group G is n_G * R_m^T C[code] / sqrt(m), so q . k_hat = sum_G n_G * sum_i
// q''_i C[code_i] with q'' = R_m q'_G / sqrt(m): the query is rotated once per head into
// every group's frame and the keys are never un-rotated.

// Prologue: q' = RoPE(q, pos) (fp64 angles), then q'' per storage position, scaled by
// softmax_scale * log2(e) / sqrt(m) so that logits come out in base-2 units.
template <typename T>
__global__ __launch_bounds__(128) void k_decode_prep(DecodeArgs a) {
  __shared__ float qs[BGTQ_MAX_HEAD_DIM];
  const int h = blockIdx.x, s = blockIdx.y;
  const int hk = h / a.group, hl = h % a.group;
  const int d = a.d, n = d / 2;
  const int64_t pos = a.q_pos ? a.q_pos[s] : int64_t(a.lengths[s]) - 1;
  const T* q = static_cast<const T*>(a.q) + (int64_t(s) * a.n_q + h) * d;
  for (int j = threadIdx.x; j < n; j += blockDim.x) {
    const int ca = a.pairing ? 2 * j : j, cb = a.pairing ? 2 * j + 1 : j + n;
    const float x0 = load_f(q, ca), x1 = load_f(q, cb);
    if (a.rope_theta > 0.0) {
      const double ang = fmod(double(pos) * pow(a.rope_theta, -2.0 * j / d), kTwoPi);
      double sn, cs;
      sincos(ang, &sn, &cs);
      qs[ca] = float(double(x0) * cs - double(x1) * sn);
      qs[cb] = float(double(x0) * sn + double(x1) * cs);
    } else {
      qs[ca] = x0;
      qs[cb] = x1;
    }
  }
  __syncthreads();
  const HeadLayout& L = a.layouts[int64_t(s) * a.n_kv + hk];
  float* dst = a.qrot + (int64_t(s) * a.n_kv + hk) * d * kQPad;
  for (int p = threadIdx.x; p < d; p += blockDim.x) {
    float v = 0.0f;
    if (p < L.d_eff) {
      const int g = L.group[p], m = L.g_m[g], first = L.g_first[g];
      const float* R = a.rot_bank + bank_offset(m) + size_t(p - first) * m;
      float acc = 0.0f;
      for (int k = 0; k < m; ++k) acc = fmaf(R[k], qs[L.perm[first + k]], acc);
      v = acc * (a.scale * kLog2e / sqrtf(float(m)));
    }
    dst[p * kQPad + hl] = v;
  }
}

// Split-K pass.  Workgroup = (split, KV head, sequence) over a contiguous range of 64-token
// tiles; each wavefront takes every nwaves-th tile and keeps its own online-softmax state.
// Keys: lane = token slot; the rotated query sits in scalar registers, the lane decodes
// its token's codes from its K record staged in LDS and accumulates the G logits.
// Values: lane = rotated coordinate; the 64 slots' codes of a coordinate are one
// contiguous segment; p * n_v per slot is broadcast from LDS.
template <int D, int MAXG>
__global__ __launch_bounds__(256) void k_decode_split(DecodeArgs a) {
  constexpr int CPL = D / 64;
  extern __shared__ uint32_t smem[];
  const int split = blockIdx.x, hk = blockIdx.y, s = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nwaves = blockDim.x >> 6;
  const int len = a.lengths[s];
  const int tiles = (len + kTile - 1) / kTile;
  const int per = (tiles + a.n_split - 1) / a.n_split;
  const int t0 = split * per;
  const int t1 = t0 + per < tiles ? t0 + per : tiles;
  const int bv = a.v_bits, chunks = a.chunks;
  const int RS = 4 * chunks + 1, VS = 2 * bv + 1;
  const int kbuf_words = 64 * RS > D * VS ? 64 * RS : D * VS;
  const int wave_words = kbuf_words + 64 * kMaxGroups + 64 * MAXG;

  float* cbk = reinterpret_cast<float*>(smem);     // [510] codebooks of widths 1..8
  float* cbv = cbk + 512;                          // [256] value codebook
  uint32_t* wbase = smem + 768 + wave * wave_words;
  uint32_t* kbuf = wbase;
  float* knorm = reinterpret_cast<float*>(wbase + kbuf_words);  // [8][64]
  float* pv = knorm + 64 * kMaxGroups;                          // [64][MAXG]

  for (int i = tid; i < 510; i += blockDim.x) {
    const int w = 31 - __clz(i + 2);
    cbk[i] = c_cen[w - 1][i + 2 - (1 << w)];
  }
  for (int i = tid; i < (1 << bv); i += blockDim.x) cbv[i] = c_cen[bv - 1][i];
  __syncthreads();

  cLayout* L = (cLayout*)(a.layouts + int64_t(s) * a.n_kv + hk);
  const int ng = L->n_groups;
  cfloat* qbase = (cfloat*)(a.qrot + (int64_t(s) * a.n_kv + hk) * D * kQPad);
  const size_t reg = size_t(s) * a.n_kv + hk;
  const int64_t cap_tiles = a.capacity / kTile;
  const uint4* kc = reinterpret_cast<const uint4*>(a.k_codes) + reg * cap_tiles * chunks * kTile;
  const uint16_t* kn = a.k_norms + reg * cap_tiles * kMaxGroups * kTile;
  const uint32_t* vc = reinterpret_cast<const uint32_t*>(a.v_codes) + reg * cap_tiles * D * 2 * bv;
  const uint16_t* vn = a.v_norms + reg * cap_tiles * kTile;

  float m[MAXG], lsum[MAXG], acc[MAXG][CPL];
#pragma unroll
  for (int h = 0; h < MAXG; ++h) {
    m[h] = -INFINITY;
    lsum[h] = 0.0f;
#pragma unroll
    for (int i = 0; i < CPL; ++i) acc[h][i] = 0.0f;
  }
  const uint32_t vmask = (1u << bv) - 1u;

  for (int tile = t0 + wave; tile < t1; tile += nwaves) {
    const int valid = len - tile * kTile < kTile ? len - tile * kTile : kTile;
    // ---- keys: stage this lane's record and group norms
    for (int c = 0; c < chunks; ++c) {
      const uint4 v = kc[(size_t(tile) * chunks + c) * kTile + lane];
      uint32_t* row = kbuf + lane * RS + 4 * c;
      row[0] = v.x; row[1] = v.y; row[2] = v.z; row[3] = v.w;
    }
    kbuf[lane * RS + 4 * chunks] = 0u;
    for (int g = 0; g < ng; ++g)
      knorm[g * 64 + lane] = f16_bits_to_f32(kn[(size_t(tile) * kMaxGroups + g) * kTile + lane]);
    float sc[MAXG];
#pragma unroll
    for (int h = 0; h < MAXG; ++h) sc[h] = 0.0f;
    for (int g = 0; g < ng; ++g) {
      const int w = L->g_width[g], first = L->g_first[g], mg = L->g_m[g], bo = L->g_bitoff[g];
      const float* cb = cbk + (1 << w) - 2;
      const uint32_t mask = (1u << w) - 1u;
      float part[MAXG];
#pragma unroll
      for (int h = 0; h < MAXG; ++h) part[h] = 0.0f;
      for (int i = 0; i < mg; ++i) {
        const int off = bo + i * w;
        const int dw = off >> 5, sh = off & 31;
        const uint32_t code = __builtin_amdgcn_alignbit(kbuf[lane * RS + dw + 1], kbuf[lane * RS + dw], sh) & mask;
        const float val = cb[code];
        cfloat* qr = qbase + size_t(first + i) * kQPad;
#pragma unroll
        for (int h = 0; h < MAXG; ++h) part[h] = fmaf(qr[h], val, part[h]);
      }
      const float nv = knorm[g * 64 + lane];
#pragma unroll
      for (int h = 0; h < MAXG; ++h) sc[h] = fmaf(nv, part[h], sc[h]);
    }
    if (lane >= valid) {
#pragma unroll
      for (int h = 0; h < MAXG; ++h) sc[h] = -INFINITY;
    }
    if (a.logits && lane < valid) {
      for (int h = 0; h < a.group; ++h)
        a.logits[(int64_t(s) * a.n_q + hk * a.group + h) * a.capacity + int64_t(tile) * kTile + lane] = sc[h] * kLn2;
    }
    // ---- online softmax (base 2)
    const float vnv = lane < valid ? f16_bits_to_f32(vn[size_t(tile) * kTile + lane]) : 0.0f;
#pragma unroll
    for (int h = 0; h < MAXG; ++h) {
      const float mn = fmaxf(m[h], wave_max(sc[h]));
      const float alpha = exp2f(m[h] - mn);
      const float p = exp2f(sc[h] - mn);
      lsum[h] = lsum[h] * alpha + p;
      m[h] = mn;
#pragma unroll
      for (int i = 0; i < CPL; ++i) acc[h][i] *= alpha;
      pv[lane * MAXG + h] = p * vnv;
    }
    wave_sync();
    // ---- values: lane = rotated coordinate
    const uint32_t* vt = vc + size_t(tile) * D * 2 * bv;
    for (int idx = lane; idx < D * 2 * bv; idx += 64) {
      const int r = idx / (2 * bv);
      kbuf[r * VS + (idx - r * 2 * bv)] = vt[idx];
    }
    for (int r = lane; r < D; r += 64) kbuf[r * VS + 2 * bv] = 0u;
    wave_sync();
    for (int t = 0; t < valid; ++t) {
      float pvals[MAXG];
#pragma unroll
      for (int h = 0; h < MAXG; ++h) pvals[h] = pv[t * MAXG + h];
      const int off = t * bv;
      const int dw = off >> 5, sh = off & 31;
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const int r = lane + 64 * i;
        const uint32_t code = __builtin_amdgcn_alignbit(kbuf[r * VS + dw + 1], kbuf[r * VS + dw], sh) & vmask;
        const float val = cbv[code];
#pragma unroll
        for (int h = 0; h < MAXG; ++h) acc[h][i] = fmaf(pvals[h], val, acc[h][i]);
      }
    }
    wave_sync();
  }

  // ---- merge the wavefronts of this workgroup, one query head at a time
#pragma unroll
  for (int h = 0; h < MAXG; ++h) lsum[h] = wave_sum(lsum[h]);
  __syncthreads();
  float* comb = reinterpret_cast<float*>(smem + 768);   // [nwaves][D + 2]
  for (int h = 0; h < a.group; ++h) {
    float ah[CPL], mh = -INFINITY, lh = 0.0f;
#pragma unroll
    for (int hh = 0; hh < MAXG; ++hh) {
      if (hh == h) {
        mh = m[hh];
        lh = lsum[hh];
#pragma unroll
        for (int i = 0; i < CPL; ++i) ah[i] = acc[hh][i];
      }
    }
#pragma unroll
    for (int i = 0; i < CPL; ++i) comb[wave * (D + 2) + lane + 64 * i] = ah[i];
    if (lane == 0) {
      comb[wave * (D + 2) + D] = mh;
      comb[wave * (D + 2) + D + 1] = lh;
    }
    __syncthreads();
    float mmax = -INFINITY;
    for (int w = 0; w < nwaves; ++w) mmax = fmaxf(mmax, comb[w * (D + 2) + D]);
    float* dst = a.partial + ((int64_t(s) * a.n_q + hk * a.group + h) * a.n_split + split) * (D + 2);
    for (int c = tid; c < D + 2; c += blockDim.x) {
      float v = 0.0f;
      if (c == D) {
        v = mmax;
      } else if (mmax != -INFINITY) {
        const int src = c == D + 1 ? D + 1 : c;
        for (int w = 0; w < nwaves; ++w) {
          const float mw = comb[w * (D + 2) + D];
          if (mw != -INFINITY) v += comb[w * (D + 2) + src] * exp2f(mw - mmax);
        }
      }
      dst[c] = v;
    }
    __syncthreads();
  }
}

// Merge the splits of one query head and undo the value rotation:
// out = R_v^T acc / (sqrt(d) * l), acc = sum_t p_t n_v,t C[code_t].
template <int D>
__global__ __launch_bounds__(256) void k_decode_combine(DecodeArgs a) {
  __shared__ float red[256];
  __shared__ float accs[D];
  __shared__ float wts[1024];
  const int h = blockIdx.x, s = blockIdx.y, tid = threadIdx.x;
  const float* part = a.partial + (int64_t(s) * a.n_q + h) * a.n_split * (D + 2);
  float mloc = -INFINITY;
  for (int i = tid; i < a.n_split; i += blockDim.x) mloc = fmaxf(mloc, part[i * (D + 2) + D]);
  red[tid] = mloc;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (tid < o) red[tid] = fmaxf(red[tid], red[tid + o]);
    __syncthreads();
  }
  const float mmax = red[0];
  __syncthreads();
  float lloc = 0.0f;
  for (int i = tid; i < a.n_split; i += blockDim.x) {
    const float mi = part[i * (D + 2) + D];
    const float w = (mi == -INFINITY) ? 0.0f : exp2f(mi - mmax);
    wts[i] = w;
    lloc += w * part[i * (D + 2) + D + 1];
  }
  red[tid] = lloc;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (tid < o) red[tid] += red[tid + o];
    __syncthreads();
  }
  const float ltot = red[0];
  for (int r = tid; r < D; r += blockDim.x) {
    float v = 0.0f;
    for (int i = 0; i < a.n_split; ++i) v = fmaf(wts[i], part[i * (D + 2) + r], v);
    accs[r] = v;
  }
  __syncthreads();
  const float inv = (ltot > 0.0f) ? 1.0f / (ltot * sqrtf(float(D))) : 0.0f;
  float* o = a.out + (int64_t(s) * a.n_q + h) * D;
  for (int j = tid; j < D; j += blockDim.x) {
    float v = 0.0f;
    for (int r = 0; r < D; ++r) v = fmaf(a.rot_v[r * D + j], accs[r], v);
    o[j] = v * inv;
  }
}

template <int D>
hipError_t launch_decode_d(const DecodeArgs& a, bgtq_dtype q_dt, hipStream_t st) {
  if (q_dt == BGTQ_BF16)
    hipLaunchKernelGGL(k_decode_prep<uint16_t>, dim3(a.n_q, a.batch), dim3(128), 0, st, a);
  else
    hipLaunchKernelGGL(k_decode_prep<float>, dim3(a.n_q, a.batch), dim3(128), 0, st, a);
  const int maxg = a.group <= 1 ? 1 : a.group <= 2 ? 2 : a.group <= 4 ? 4 : a.group <= 8 ? 8 : 16;
  const int RS = 4 * a.chunks + 1, VS = 2 * a.v_bits + 1;
  const int kbuf_words = 64 * RS > D * VS ? 64 * RS : D * VS;
  const int wave_words = kbuf_words + 64 * kMaxGroups + 64 * maxg;
  int nwaves = 4;
  while (nwaves > 1 && (768 + nwaves * wave_words) * 4 > 64 * 1024) --nwaves;
  const size_t lds = size_t(768 + nwaves * wave_words) * 4;
  const dim3 grid(a.n_split, a.n_kv, a.batch), block(64 * nwaves);
  switch (maxg) {
    case 1: hipLaunchKernelGGL((k_decode_split<D, 1>), grid, block, lds, st, a); break;
    case 2: hipLaunchKernelGGL((k_decode_split<D, 2>), grid, block, lds, st, a); break;
    case 4: hipLaunchKernelGGL((k_decode_split<D, 4>), grid, block, lds, st, a); break;
    case 8: hipLaunchKernelGGL((k_decode_split<D, 8>), grid, block, lds, st, a); break;
    default: hipLaunchKernelGGL((k_decode_split<D, 16>), grid, block, lds, st, a); break;
  }
  hipLaunchKernelGGL(k_decode_combine<D>, dim3(a.n_q, a.batch), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace

// ===================================================================== launchers

hipError_t upload_tables(const Tables& t) {
  hipError_t e = hipMemcpyToSymbol(HIP_SYMBOL(c_thr), t.thr, sizeof(t.thr));
  if (e == hipSuccess) e = hipMemcpyToSymbol(HIP_SYMBOL(c_cen), t.cen, sizeof(t.cen));
  if (e == hipSuccess) e = hipMemcpyToSymbol(HIP_SYMBOL(c_dgain), t.dgain, sizeof(t.dgain));
  return e;
}

hipError_t launch_energy(const void* keys, bgtq_dtype dt, int n_heads, int64_t n_tokens, int d, int64_t sh,
                         int64_t st, int pairing, double* energy, double* partial, hipStream_t s) {
  const int n = d / 2;
  const int n_chunks = int((n_tokens + kEnergyChunk - 1) / kEnergyChunk);
  const int64_t total = int64_t(n_heads) * n_chunks * n;
  const dim3 grid(unsigned((total + 255) / 256));
  if (dt == BGTQ_BF16)
    hipLaunchKernelGGL(k_energy_partial<uint16_t>, grid, dim3(256), 0, s, static_cast<const uint16_t*>(keys),
                       n_heads, n_tokens, n, sh, st, pairing, n_chunks, partial);
  else
    hipLaunchKernelGGL(k_energy_partial<float>, grid, dim3(256), 0, s, static_cast<const float*>(keys),
                       n_heads, n_tokens, n, sh, st, pairing, n_chunks, partial);
  hipLaunchKernelGGL(k_energy_final, dim3((n_heads * n + 255) / 256), dim3(256), 0, s, partial, n_heads,
                     n_chunks, n, n_tokens, energy);
  return hipGetLastError();
}

hipError_t launch_allocate(const double* energy, int n_heads, int n_blocks, int increments, int b_min,
                           int b_max, int pairing, uint8_t* widths, HeadLayout* layouts, hipStream_t s) {
  hipLaunchKernelGGL(k_allocate, dim3(n_heads), dim3(64), 0, s, energy, n_blocks, increments, b_min, b_max,
                     pairing, widths, layouts);
  return hipGetLastError();
}

hipError_t launch_append(const AppendArgs& a, bgtq_dtype dt, int n_seqs, hipStream_t s) {
  const int halves = int((a.n_new + kHalf - 1) / kHalf) + 1;
  const dim3 grid(halves, a.n_kv_heads, n_seqs);
  const size_t lds = size_t(kHalf) * (a.d + 1) * 4 + kMaxBits * 255 * 4 + kHalf * kMaxGroups * 4 + kHalf * 4 +
                     2 * kHalf * BGTQ_MAX_HEAD_DIM + 2 * 64 * 4;
  if (dt == BGTQ_BF16)
    hipLaunchKernelGGL(k_append<uint16_t>, grid, dim3(256), lds, s, a);
  else
    hipLaunchKernelGGL(k_append<float>, grid, dim3(256), lds, s, a);
  hipLaunchKernelGGL(k_advance, dim3((n_seqs + 63) / 64), dim3(64), 0, s, a.lengths, a.seq_begin, n_seqs, a.n_new,
                     a.capacity);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, bgtq_dtype q_dt, hipStream_t s) {
  switch (a.d) {
    case 64: return launch_decode_d<64>(a, q_dt, s);
    case 128: return launch_decode_d<128>(a, q_dt, s);
    case 256: return launch_decode_d<256>(a, q_dt, s);
    default: return hipErrorInvalidValue;
  }
}

int decode_splits(int batch, int n_kv_heads, int64_t capacity) {
  const int64_t tiles = capacity / kTile;
  const int64_t units = int64_t(batch) * n_kv_heads;
  int64_t want = (1024 + units - 1) / units;         // about 1024 workgroups in flight
  const int64_t by_work = (tiles + 7) / 8;            // at least 8 tiles per split
  if (want > by_work) want = by_work;
  if (want < 1) want = 1;
  if (want > 1024) want = 1024;
  return int(want);
}

}  // namespace bgtq
