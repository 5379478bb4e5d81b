// HIP kernels of the Block-GTQ packed-cache decode path, written for gfx950 (CDNA4, wave64).
//
// Method: "RoPE-Aware Bit Allocation for KV-Cache Quantization" (arXiv 2606.24033), abstract.
// Each kernel states the reading of the abstract it implements.  Kernels that must agree
// bit for bit with the specified arithmetic (energy, allocation, quantize-and-pack) are
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
__constant__ uint32_t c_pair[kPairWords];
__constant__ uint16_t c_single[kSingleHalves];

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
    // matrix-core view: segments of at most 8 positions in storage order; a k-step takes up to
    // 4 consecutive segments from at most two groups (the two halves of the output columns)
    int ks = -1, slot = 4, ga = -1, gb = -1;
    for (int gg = 0; gg < g; ++gg) {
      const int w = lay.g_width[gg];
      for (int s0 = 0; s0 < lay.g_m[gg]; s0 += kSegLen) {
        if (slot == 4 || (gg != ga && gg != gb && gb >= 0)) {
          if (ks >= 0) lay.kgroups[ks] = uint32_t(ga) | uint32_t(gb >= 0 ? gb : ga) << 8;
          ++ks; slot = 0; ga = gg; gb = -1;
        } else if (gg != ga && gb < 0) {
          gb = gg;
        }
        const int cnt = lay.g_m[gg] - s0 < kSegLen ? lay.g_m[gg] - s0 : kSegLen;
        const uint32_t half = gg == ga ? 0u : 1u;
        lay.seg[4 * ks + slot] = uint32_t(lay.g_bitoff[gg] + s0 * w) | uint32_t(w) << 16 | uint32_t(gg) << 20 |
                                 uint32_t(cnt) << 24 | half << 28;
        for (int e = 0; e < cnt; ++e)
          lay.kpos[lay.g_first[gg] + s0 + e] = uint16_t(32 * ks + kSegLen * slot + e);
        ++slot;
      }
    }
    if (ks >= 0) lay.kgroups[ks] = uint32_t(ga) | uint32_t(gb >= 0 ? gb : ga) << 8;
    lay.n_ksteps = ks + 1;
    // storage positions with bits in record dword w (offsets ascend with the position)
    for (int w = 0, p0 = 0, p1 = 0; w < 4 * lay.chunks; ++w) {
      while (p0 < pos && int(lay.offset[p0]) + lay.g_width[lay.group[p0]] <= 32 * w) ++p0;
      if (p1 < p0) p1 = p0;
      while (p1 < pos && int(lay.offset[p1]) < 32 * w + 32) ++p1;
      lay.dw_first[w] = uint16_t(p0);
      lay.dw_end[w] = uint16_t(p1);
    }
    for (int i = 0; i < 4 * lay.n_ksteps; ++i)
      if (lay.seg[i] == 0u) lay.seg[i] = 1u << 16;   // unused slot: width 1 at bit 0
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

// Sequential fp32 dot product sum_k R[k] * x[k] (ascending k, no fused multiply-add).  R is
// read as float2 (m is even and every row starts 8-byte aligned), 64 values per batch with
// all of a batch's loads issued before the first add, so one memory latency covers 64 terms.
__device__ __forceinline__ float seq_dot(const float* __restrict__ R, const float* x, int m) {
  const float2* R2 = reinterpret_cast<const float2*>(R);
  float acc = 0.0f;
  for (int k0 = 0; k0 < m; k0 += 64) {
    float2 r[32];
#pragma unroll
    for (int i = 0; i < 32; ++i)
      if (k0 + 2 * i < m) r[i] = R2[k0 / 2 + i];
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      if (k0 + 2 * i < m) {
        acc = acc + r[i].x * x[k0 + 2 * i];
        acc = acc + r[i].y * x[k0 + 2 * i + 1];
      }
    }
  }
  return acc;
}

template <typename T>
__global__ __launch_bounds__(256) void k_append(AppendArgs a) {
  extern __shared__ float sm[];
  const int d = a.d;
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
  const int r0 = int(lo - ht * kHalf), nrows = int(hi - lo);   // active rows r0 .. r0 + nrows - 1
  const int64_t tile = ht / 2;
  const int half = int(ht & 1);
  const int XS = d + 1;
  float* xg = sm;                                   // [32][d+1] keys in storage order
  float* xs = sm;                                   // same buffer, later: values in original order
  float* thr = xg + kHalf * XS;                     // [8][255]
  float* knrm = thr + kMaxBits * 255;               // [32][8]
  float* vnrm = knrm + kHalf * kMaxGroups;          // [32]
  uint8_t* kcode = reinterpret_cast<uint8_t*>(vnrm + kHalf);             // [32][256]
  uint8_t* vcode = kcode + kHalf * BGTQ_MAX_HEAD_DIM;                      // [32][256]
  HeadLayout* Ls = reinterpret_cast<HeadLayout*>(vcode + kHalf * BGTQ_MAX_HEAD_DIM);   // LDS copy

  {
    const uint4* src = reinterpret_cast<const uint4*>(a.layouts + int64_t(s) * a.n_kv_heads + hk);
    uint4* dst = reinterpret_cast<uint4*>(Ls);
    for (int i = tid; i < int(sizeof(HeadLayout) / 16); i += nt) dst[i] = src[i];
  }
  const HeadLayout& L = *Ls;
  __syncthreads();
  const int ng = L.n_groups, d_eff = L.d_eff, n_dw = 4 * a.chunks;
  const size_t reg = size_t(s) * a.n_kv_heads + hk;
  const int64_t tiles = a.capacity / kTile;
  // few rows (decode): spread one row's outputs over the threads; many rows: lanes run over rows
  const bool by_pos = nrows <= 4;

  for (int i = tid; i < kMaxBits * 255; i += nt) thr[i] = c_thr[i / 255][i % 255];
  const T* kin = static_cast<const T*>(a.keys) + si * a.stride_seq + hk * a.stride_head;
  const T* vin = static_cast<const T*>(a.values) + si * a.stride_seq + hk * a.stride_head;
  for (int idx = tid; idx < nrows * d_eff; idx += nt) {
    const int r = r0 + idx / d_eff, p = idx % d_eff;
    xg[r * XS + p] = load_f(kin, (ht * kHalf + r - len) * a.stride_token + L.perm[p]);
  }
  __syncthreads();
  // key group norms: sequential fp32 sum of squares in storage order
  for (int it = tid; it < nrows * ng; it += nt) {
    const int r = r0 + it % nrows, g = it / nrows;
    const float* x = xg + r * XS + L.g_first[g];
    float ss = 0.0f;
    for (int k = 0; k < L.g_m[g]; ++k) ss = ss + x[k] * x[k];
    knrm[r * kMaxGroups + g] = sqrtf(ss);
  }
  __syncthreads();
  // key codes, storage order
  for (int it = tid; it < nrows * d_eff; it += nt) {
    const int r = r0 + (by_pos ? it / d_eff : it % nrows);
    const int p = by_pos ? it % d_eff : it / nrows;
    const int g = L.group[p], w = L.g_width[g], m = L.g_m[g], first = L.g_first[g];
    const float acc = seq_dot(a.rot_bank + bank_offset(m) + size_t(p - first) * m, xg + r * XS + first, m);
    const float nv = knrm[r * kMaxGroups + g];
    int code = 0;
    if (nv != 0.0f) code = code_of(thr + (w - 1) * 255, w, (acc / nv) * sqrtf(float(m)));
    kcode[r * BGTQ_MAX_HEAD_DIM + p] = uint8_t(code);
  }
  __syncthreads();
  for (int idx = tid; idx < nrows * d; idx += nt) {
    const int r = r0 + idx / d, c = idx % d;
    xs[r * XS + c] = load_f(vin, (ht * kHalf + r - len) * a.stride_token + c);
  }
  __syncthreads();
  for (int r = r0 + tid; r < r0 + nrows; r += nt) {
    float ss = 0.0f;
    for (int k = 0; k < d; ++k) ss = ss + xs[r * XS + k] * xs[r * XS + k];
    vnrm[r] = sqrtf(ss);
  }
  __syncthreads();
  const float sd = sqrtf(float(d));
  for (int it = tid; it < nrows * d; it += nt) {
    const int r = r0 + (by_pos ? it / d : it % nrows);
    const int i = by_pos ? it % d : it / nrows;
    const float acc = seq_dot(a.rot_v + size_t(i) * d, xs + r * XS, d);
    const float nv = vnrm[r];
    int code = 0;
    if (nv != 0.0f) code = code_of(thr + (a.v_bits - 1) * 255, a.v_bits, (acc / nv) * sd);
    vcode[r * BGTQ_MAX_HEAD_DIM + i] = uint8_t(code);
  }
  __syncthreads();
  // pack key records (one thread per (slot, record dword))
  uint32_t* kc = reinterpret_cast<uint32_t*>(a.k_codes) + reg * tiles * a.chunks * kTile * 4;
  for (int it = tid; it < nrows * n_dw; it += nt) {
    const int r = r0 + it % nrows, w = it / nrows;
    const int64_t slot = ht * kHalf + r;
    uint32_t v = 0;
    for (int p = L.dw_first[w]; p < L.dw_end[w]; ++p) {
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
    const int bit0 = 32 * w;
    const int j_lo = bit0 / bv, j_hi = (bit0 + 31) / bv;
    // only dwords that hold bits of an appended slot are rewritten
    if (tile * kTile + j_hi < lo || tile * kTile + j_lo >= hi) continue;
    uint32_t v = *addr;
    for (int j = j_lo; j <= j_hi; ++j) {
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
  for (int it = tid; it < nrows * ng; it += nt) {
    const int r = r0 + it % nrows, g = it / nrows;
    const int64_t slot = ht * kHalf + r;
    kn[(tile * kMaxGroups + g) * kTile + slot % kTile] = f32_to_f16_bits(fminf(knrm[r * kMaxGroups + g], 65504.0f));
  }
  for (int r = r0 + tid; r < r0 + nrows; r += nt) {
    const int64_t slot = ht * kHalf + r;
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
// softmax_scale * log2(e) / sqrt(m) so that logits come out in base-2 units.  Written in two
// forms: fp32 [position][head] for the vector-ALU kernel and fp16 matrix-core B operands
// [k-step][lane][8] for the MFMA kernel (k index 32 s + 8 j + e lives in lane 16 j + head).
template <typename T>
__global__ __launch_bounds__(128) void k_decode_prep(DecodeArgs a) {
  __shared__ float qs[BGTQ_MAX_HEAD_DIM];
  __shared__ float qk[32 * kMaxKSteps];
  const int h = blockIdx.x, s = blockIdx.y;
  const int hk = h / a.group, hl = h % a.group;
  const int d = a.d, n = d / 2;
  const int64_t pos = a.q_pos ? a.q_pos[s] : int64_t(a.lengths[s]) - 1;
  const T* q = static_cast<const T*>(a.q) + (int64_t(s) * a.n_q + h) * d;
  for (int j = threadIdx.x; j < n; j += blockDim.x) {
    const int ca = a.pairing ? 2 * j : j, cb = a.pairing ? 2 * j + 1 : j + n;
    const float x0 = load_f(q, ca), x1 = load_f(q, cb);
    if (a.rope_theta > 0.0) {
      const double ang = fmod(double(pos) * a.inv_freq[j], kTwoPi);
      double sn, cs;
      sincos(ang, &sn, &cs);
      qs[ca] = float(double(x0) * cs - double(x1) * sn);
      qs[cb] = float(double(x0) * sn + double(x1) * cs);
    } else {
      qs[ca] = x0;
      qs[cb] = x1;
    }
  }
  for (int i = threadIdx.x; i < 32 * kMaxKSteps; i += blockDim.x) qk[i] = 0.0f;
  __syncthreads();
  const HeadLayout& L = a.layouts[int64_t(s) * a.n_kv + hk];
  float* dst = a.qrot + (int64_t(s) * a.n_kv + hk) * d * kQPad;
  for (int p = threadIdx.x; p < d; p += blockDim.x) {
    float v = 0.0f;
    if (p < L.d_eff) {
      const int g = L.group[p], m = L.g_m[g], first = L.g_first[g];
      const float2* R2 = reinterpret_cast<const float2*>(a.rot_bank + bank_offset(m) + size_t(p - first) * m);
      float acc = 0.0f;
      for (int k0 = 0; k0 < m; k0 += 64) {
        float2 r[32];
#pragma unroll
        for (int i = 0; i < 32; ++i)
          if (k0 + 2 * i < m) r[i] = R2[k0 / 2 + i];
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          if (k0 + 2 * i < m) {
            acc = fmaf(r[i].x, qs[L.perm[first + k0 + 2 * i]], acc);
            acc = fmaf(r[i].y, qs[L.perm[first + k0 + 2 * i + 1]], acc);
          }
        }
      }
      v = acc * (a.scale * kLog2e / sqrtf(float(m)));
      qk[L.kpos[p]] = v;
    }
    dst[p * kQPad + hl] = v;
  }
  __syncthreads();
  // matrix-core B operands: lane 16 j + c of k-step ks holds k indices 32 ks + 8 j + e; column
  // c < 8 carries head c for the k-step's first group, column c + 8 head c for its second
  // group; each value is split into an fp16 high part and an fp16 remainder.
  if (!a.use_mfma) return;   // the matrix-core kernel is used only for group sizes <= 8
  uint16_t* qm = a.qmma + (int64_t(s) * a.n_kv + hk) * kMaxKSteps * 2 * 64 * 8;
  const int nk = L.n_ksteps * 32;
  for (int i = threadIdx.x; i < nk; i += blockDim.x) {
    const int ks = i / 32, jj = (i / 8) % 4, e = i % 8;
    const uint32_t half = (L.seg[4 * ks + jj] >> 28) & 1u;
    const float v = qk[i];
    const uint16_t vh = f32_to_f16_bits(v);
    const uint16_t vl = f32_to_f16_bits(v - f16_bits_to_f32(vh));
    const int lane_on = jj * 16 + hl + 8 * int(half), lane_off = jj * 16 + hl + 8 * int(1u - half);
    qm[((ks * 2 + 0) * 64 + lane_on) * 8 + e] = vh;
    qm[((ks * 2 + 1) * 64 + lane_on) * 8 + e] = vl;
    qm[((ks * 2 + 0) * 64 + lane_off) * 8 + e] = 0;
    qm[((ks * 2 + 1) * 64 + lane_off) * 8 + e] = 0;
  }
  if (hl == 0) {  // columns of absent query heads stay zero
    const int pad = 8 - a.group;
    for (int i = threadIdx.x; i < nk * 2 * pad; i += blockDim.x) {
      const int c = a.group + i % pad, rest = i / pad;
      const int k = rest % nk, part = rest / nk;     // part: 0..1 = column half
      const int ks = k / 32, jj = (k / 8) % 4, e = k % 8;
      qm[((ks * 2 + 0) * 64 + jj * 16 + c + 8 * part) * 8 + e] = 0;
      qm[((ks * 2 + 1) * 64 + jj * 16 + c + 8 * part) * 8 + e] = 0;
    }
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
    cbk[i] = f16_bits_to_f32(f32_to_f16_bits(c_cen[w - 1][i + 2 - (1 << w)]));   // fp16 levels
  }
  for (int i = tid; i < (1 << bv); i += blockDim.x) cbv[i] = f16_bits_to_f32(f32_to_f16_bits(c_cen[bv - 1][i]));
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

// ---------------------------------------------------------------- matrix-core split-K pass
// Same partial results as k_decode_split, with both contractions on MFMA (v_mfma_f32_16x16x32_f16).
//   Keys: S^T[token][head] = K_hat[token][k] * Q''[k][head].  A rows are 16 tokens, the k axis
//   is the head's width groups cut into 8-position segments (lane group j = lane / 16 decodes
//   segment 4 s + j of k-step s from the token's K record staged in LDS), B is the resident
//   rotated query (16 columns; columns >= G are zero).  A holds C[code] * n_group in fp16.
//   Rows of M-tile mt of sub-tile st are tokens 32 st + 8 (m / 4) + 4 mt + m % 4, so each lane
//   ends with 8 consecutive tokens of one head -- exactly the B operand layout of P V.
//   Values: acc^T[coord][head] += V_hat^T[coord][token] * P'^T[token][head], P' = p * n_v; A
//   rows are coordinates, each lane decodes 8 consecutive tokens of one coordinate from the
//   tile's coordinate-major value segment (staged in LDS).
//   Codes become fp16 through pair tables (two codes of width w <= 5 index one packed half2).
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kSegWords = 4 * kMaxKSteps + kMaxKSteps + 2;       // staged seg[] and kgroups[], 16-byte rounded
constexpr int kTableWords = kPairWords + kSingleHalves / 2 + ((kSegWords + 3) & ~3);

__device__ __forceinline__ int pair_base(int w) { return ((1 << (2 * w)) - 4) / 3; }

// Per-wave LDS words of the matrix-core kernel (K records, norms, value segments; reused for
// the final merge), rounded to 16 bytes.
__host__ __device__ inline int mfma_region_words(int D, int RS, int VS) {
  const int stage = 64 * RS + 64 * kMaxGroups + D * VS;
  const int merge = 16 * (D + 2);
  return ((stage > merge ? stage : merge) + 3) & ~3;
}
__device__ __forceinline__ int single_base(int w) { return w == 6 ? 0 : (w == 7 ? 64 : 192); }

// Eight consecutive codes of width w starting at bit `sh` of the 96-bit window (d2:d1:d0),
// decoded to fp16 reconstruction levels (low half = first code).
__device__ __forceinline__ u32x4 decode8(uint32_t d0, uint32_t d1, uint32_t d2, int sh, int w,
                                         const uint32_t* ptab, const uint16_t* stab) {
  const uint32_t lo = __builtin_amdgcn_alignbit(d1, d0, sh);
  const uint32_t hi = __builtin_amdgcn_alignbit(d2, d1, sh);
  const uint64_t x = (uint64_t(hi) << 32) | lo;
  u32x4 r;
  if (w <= 5) {
    const uint32_t* t = ptab + pair_base(w);
    const uint32_t mask = (1u << (2 * w)) - 1u;
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) r[e2] = t[uint32_t(x >> (2 * e2 * w)) & mask];
  } else {
    const uint16_t* t = stab + single_base(w);
    const uint32_t mask = (1u << w) - 1u;
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
      const uint32_t c0 = uint32_t(x >> (2 * e2 * w)) & mask;
      const uint32_t c1 = uint32_t(x >> ((2 * e2 + 1) * w)) & mask;
      r[e2] = uint32_t(t[c0]) | (uint32_t(t[c1]) << 16);
    }
  }
  return r;
}

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_decode_mfma(DecodeArgs a) {
  constexpr int MT = D / 16;
  extern __shared__ uint32_t smem[];
  const int split = blockIdx.x, hk = blockIdx.y, s = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nwaves = blockDim.x >> 6;
  const int n = lane & 15, j = lane >> 4;
  const int len = a.lengths[s];
  const int tiles = (len + kTile - 1) / kTile;
  const int per = (tiles + a.n_split - 1) / a.n_split;
  const int t0 = split * per;
  const int t1 = t0 + per < tiles ? t0 + per : tiles;
  const int bv = a.v_bits, chunks = a.chunks;
  const int RS = 4 * chunks + 3, VS = 2 * bv + 3;
  const int region_words = mfma_region_words(D, RS, VS);

  uint32_t* ptab = smem;
  uint16_t* stab = reinterpret_cast<uint16_t*>(smem + kPairWords);
  uint32_t* krec = smem + kTableWords + wave * region_words;   // [64][RS]
  float* knorm = reinterpret_cast<float*>(krec + 64 * RS);       // [8][64] fp32 group norms
  uint32_t* vseg = krec + 64 * RS + 64 * kMaxGroups;            // [D][VS]

  uint32_t* lseg = smem + kPairWords + kSingleHalves / 2;        // [4 * kMaxKSteps] then kgroups
  uint32_t* lkg = lseg + 4 * kMaxKSteps;
  const HeadLayout* L = a.layouts + int64_t(s) * a.n_kv + hk;
  for (int i = tid; i < kPairWords; i += blockDim.x) ptab[i] = c_pair[i];
  for (int i = tid; i < kSingleHalves; i += blockDim.x) stab[i] = c_single[i];
  for (int i = tid; i < 4 * kMaxKSteps; i += blockDim.x) lseg[i] = L->seg[i];
  for (int i = tid; i < kMaxKSteps; i += blockDim.x) lkg[i] = L->kgroups[i];
  __syncthreads();

  const int ng = L->n_groups, nks = L->n_ksteps;
  const uint4* qm = reinterpret_cast<const uint4*>(a.qmma + (int64_t(s) * a.n_kv + hk) * kMaxKSteps * 2 * 64 * 8);
  const size_t reg = size_t(s) * a.n_kv + hk;
  const int64_t cap_tiles = a.capacity / kTile;
  const uint4* kc = reinterpret_cast<const uint4*>(a.k_codes) + reg * cap_tiles * chunks * kTile;
  const uint16_t* kn = a.k_norms + reg * cap_tiles * kMaxGroups * kTile;
  const uint32_t* vc = reinterpret_cast<const uint32_t*>(a.v_codes) + reg * cap_tiles * D * 2 * bv;
  const uint16_t* vn = a.v_norms + reg * cap_tiles * kTile;

  f32x4 acc[MT];
#pragma unroll
  for (int mi = 0; mi < MT; ++mi) acc[mi] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.0f;
  const bool real_col = n < 8 && n < a.group;   // output column n carries query head n

  for (int tile = t0 + wave; tile < t1; tile += nwaves) {
    const int valid = len - tile * kTile < kTile ? len - tile * kTile : kTile;
    // ---- stage the tile: K records and group norms (lane = slot), value segments (lane =
    // coordinate row).  All loads of the tile are issued before the first LDS write.
    {
      constexpr int MAXCH = D / 16;                 // record chunks at 8 bits per coordinate
      constexpr int MAXVW = 8;                      // 8-byte words per value segment (8 bits)
      constexpr int RPL = D / 64;                   // value rows per lane
      uint4 kr[MAXCH];
      uint16_t knv[kMaxGroups];
      uint2 vr[RPL][MAXVW];
#pragma unroll
      for (int c = 0; c < MAXCH; ++c)
        if (c < chunks) kr[c] = kc[(size_t(tile) * chunks + c) * kTile + lane];
#pragma unroll
      for (int g = 0; g < kMaxGroups; ++g)
        if (g < ng) knv[g] = kn[(size_t(tile) * kMaxGroups + g) * kTile + lane];
      const uint2* vt2 = reinterpret_cast<const uint2*>(vc + size_t(tile) * D * 2 * bv);
#pragma unroll
      for (int i = 0; i < RPL; ++i)
#pragma unroll
        for (int wv = 0; wv < MAXVW; ++wv)
          if (wv < bv) vr[i][wv] = vt2[(lane + 64 * i) * bv + wv];
#pragma unroll
      for (int c = 0; c < MAXCH; ++c) {
        if (c < chunks) {
          uint32_t* row = krec + lane * RS + 4 * c;
          row[0] = kr[c].x; row[1] = kr[c].y; row[2] = kr[c].z; row[3] = kr[c].w;
        }
      }
      krec[lane * RS + 4 * chunks] = 0u;
      krec[lane * RS + 4 * chunks + 1] = 0u;
      krec[lane * RS + 4 * chunks + 2] = 0u;
#pragma unroll
      for (int g = 0; g < kMaxGroups; ++g)
        if (g < ng) knorm[g * 64 + lane] = f16_bits_to_f32(knv[g]);
#pragma unroll
      for (int i = 0; i < RPL; ++i) {
        uint32_t* row = vseg + (lane + 64 * i) * VS;
#pragma unroll
        for (int wv = 0; wv < MAXVW; ++wv) {
          if (wv < bv) { row[2 * wv] = vr[i][wv].x; row[2 * wv + 1] = vr[i][wv].y; }
        }
        row[2 * bv] = 0u;
        row[2 * bv + 1] = 0u;
        row[2 * bv + 2] = 0u;
      }
    }
    wave_sync();

    // ---- logits: per k-step two MFMAs (query high part, remainder) per 16-token M-tile; the
    // k-step's group partials are scaled by fp32 norms.  M-tile M = 2 st + mt has row m as
    // token 32 st + 8 (m / 4) + 4 mt + m % 4; output rows 4 j + r are tokens 32 st + 8 j + 4 mt + r.
    f32x4 S[4];
#pragma unroll
    for (int M = 0; M < 4; ++M) S[M] = f32x4{0.f, 0.f, 0.f, 0.f};
    uint4 qh_next = nks > 0 ? qm[lane] : uint4{0u, 0u, 0u, 0u};
    uint4 ql_next = nks > 0 ? qm[64 + lane] : uint4{0u, 0u, 0u, 0u};
#pragma unroll 1
    for (int ks = 0; ks < nks; ++ks) {
      const f16x8 qh = __builtin_bit_cast(f16x8, qh_next);
      const f16x8 ql = __builtin_bit_cast(f16x8, ql_next);
      if (ks + 1 < nks) {   // prefetch the next k-step's query operands
        qh_next = qm[((ks + 1) * 2 + 0) * 64 + lane];
        ql_next = qm[((ks + 1) * 2 + 1) * 64 + lane];
      }
      const uint32_t desc = lseg[4 * ks + j];
      const uint32_t kg = lkg[ks];
      const int ngrp = n < 8 ? int(kg & 0xff) : int((kg >> 8) & 0xff);
      const int w = (desc >> 16) & 15, o = desc & 0xffff;
      const int sh = o & 31;
      const uint32_t* krow0 = krec + (o >> 5);
      // the lane's window of its four tokens' records
      uint32_t d0[4], d1[4];
#pragma unroll
      for (int M = 0; M < 4; ++M) {
        const uint32_t* row = krow0 + (32 * (M >> 1) + 8 * (n >> 2) + 4 * (M & 1) + (n & 3)) * RS;
        d0[M] = row[0];
        d1[M] = row[1];
      }
      u32x4 raw[4];
      if (w <= 4) {   // 8 codes fit one 32-bit window: one bit-field extract per pair
        const uint32_t* t = ptab + pair_base(w);
#pragma unroll
        for (int M = 0; M < 4; ++M) {
          const uint32_t x = __builtin_amdgcn_alignbit(d1[M], d0[M], sh);
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) raw[M][e2] = t[__builtin_amdgcn_ubfe(x, 2 * e2 * w, 2 * w)];
        }
      } else {
#pragma unroll
        for (int M = 0; M < 4; ++M) {
          const uint32_t* row = krow0 + (32 * (M >> 1) + 8 * (n >> 2) + 4 * (M & 1) + (n & 3)) * RS;
          raw[M] = decode8(d0[M], d1[M], row[2], sh, w, ptab, stab);
        }
      }
#pragma unroll
      for (int M = 0; M < 4; ++M) {
        const f16x8 A = __builtin_bit_cast(f16x8, raw[M]);
        f32x4 T = {0.f, 0.f, 0.f, 0.f};
        T = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, qh, T, 0, 0, 0);
        T = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, ql, T, 0, 0, 0);
        const float4 nv = *reinterpret_cast<const float4*>(knorm + ngrp * 64 + 32 * (M >> 1) + 8 * j + 4 * (M & 1));
        S[M][0] = fmaf(T[0], nv.x, S[M][0]);
        S[M][1] = fmaf(T[1], nv.y, S[M][1]);
        S[M][2] = fmaf(T[2], nv.z, S[M][2]);
        S[M][3] = fmaf(T[3], nv.w, S[M][3]);
      }
    }
    // head c's logit = column c + column c + 8 (lanes n and n ^ 8 of the same row)
#pragma unroll
    for (int M = 0; M < 4; ++M) {
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = S[M][r];
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] += __shfl_xor(v[r], 8);
#pragma unroll
      for (int r = 0; r < 4; ++r) S[M][r] = v[r];
    }

    // ---- per 32-token sub-tile: online softmax (base 2), then P V on the matrix cores
#pragma unroll 1
    for (int st = 0; st < 2; ++st) {
      if (32 * st >= valid) break;
      float sv[8];
      float tmax = -INFINITY;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = st == 0 ? S[e >> 2][e & 3] : S[2 + (e >> 2)][e & 3];
        sv[e] = (32 * st + 8 * j + e < valid) ? x : -INFINITY;
        tmax = fmaxf(tmax, sv[e]);
      }
      if (a.logits && real_col) {
        float* lg = a.logits + (int64_t(s) * a.n_q + hk * a.group + n) * a.capacity + int64_t(tile) * kTile +
                    32 * st + 8 * j;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (32 * st + 8 * j + e < valid) lg[e] = sv[e] * kLn2;
      }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
      const float mn = fmaxf(m_run, tmax);
      const float alpha = exp2f(m_run - mn);
      m_run = mn;
      const uint4 nvraw = *reinterpret_cast<const uint4*>(vn + size_t(tile) * kTile + 32 * st + 8 * j);
      const f16x8 nvv = __builtin_bit_cast(f16x8, nvraw);
      float psum = 0.0f;
      f16x8 bp;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p = exp2f(sv[e] - mn);
        psum += p;
        bp[e] = (_Float16)((real_col && 32 * st + 8 * j + e < valid) ? p * float(nvv[e]) : 0.0f);
      }
      l_run = l_run * alpha + psum;
      if (__any(alpha != 1.0f)) {   // the running maxima moved: rescale the accumulators
#pragma unroll
        for (int mi = 0; mi < MT; ++mi) acc[mi] *= alpha;
      }
      const int start = (32 * st + 8 * j) * bv;
      const int wofs = start >> 5, sh = start & 31;
      const uint32_t* vrow0 = vseg + n * VS + wofs;
      if (bv <= 4) {   // uniform: 8 codes per 32-bit window, pair fields at fixed offsets
        const uint32_t* t = ptab + pair_base(bv);
        uint32_t x[MT];
#pragma unroll
        for (int mi = 0; mi < MT; ++mi) {
          const uint32_t* row = vrow0 + 16 * mi * VS;
          x[mi] = __builtin_amdgcn_alignbit(row[1], row[0], sh);
        }
#pragma unroll
        for (int mi = 0; mi < MT; ++mi) {
          u32x4 raw;
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) raw[e2] = t[__builtin_amdgcn_ubfe(x[mi], 2 * e2 * bv, 2 * bv)];
          acc[mi] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, raw), bp, acc[mi], 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int mi = 0; mi < MT; ++mi) {
          const uint32_t* row = vrow0 + 16 * mi * VS;
          const u32x4 raw = decode8(row[0], row[1], row[2], sh, bv, ptab, stab);
          acc[mi] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, raw), bp, acc[mi], 0, 0, 0);
        }
      }
    }
    wave_sync();
  }

  // ---- merge the wavefronts of this workgroup: lane (n, j) holds head n, coords 16 mi + 4 j + r
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  __syncthreads();
  float* comb = reinterpret_cast<float*>(smem + kTableWords) + wave * region_words;   // [16][D + 2]
#pragma unroll
  for (int mi = 0; mi < MT; ++mi)
#pragma unroll
    for (int r = 0; r < 4; ++r) comb[n * (D + 2) + 16 * mi + 4 * j + r] = acc[mi][r];
  if (j == 0) {
    comb[n * (D + 2) + D] = m_run;
    comb[n * (D + 2) + D + 1] = l_run;
  }
  __syncthreads();
  const float* comb0 = reinterpret_cast<const float*>(smem + kTableWords);
  for (int item = tid; item < a.group * (D + 2); item += blockDim.x) {
    const int hh = item / (D + 2), c = item % (D + 2);
    float mmax = -INFINITY;
    for (int w = 0; w < nwaves; ++w) mmax = fmaxf(mmax, comb0[w * region_words + hh * (D + 2) + D]);
    float v = 0.0f;
    if (c == D) {
      v = mmax;
    } else if (mmax != -INFINITY) {
      for (int w = 0; w < nwaves; ++w) {
        const float mw = comb0[w * region_words + hh * (D + 2) + D];
        if (mw != -INFINITY) v += comb0[w * region_words + hh * (D + 2) + c] * exp2f(mw - mmax);
      }
    }
    a.partial[((int64_t(s) * a.n_q + hk * a.group + hh) * a.n_split + split) * (D + 2) + c] = v;
  }
}

// Merge the splits of one query head and undo the value rotation:
// out = R_v^T acc / (sqrt(d) * l), acc = sum_t p_t n_v,t C[code_t].  1024 threads: NSUB
// threads share a coordinate, each over every NSUB-th split, so many loads are in flight.
template <int D>
__global__ __launch_bounds__(1024) void k_decode_combine(DecodeArgs a) {
  constexpr int NT = 1024, NSUB = NT / D;
  __shared__ float red[NT];
  __shared__ float accs[D];
  __shared__ float wts[1024];
  const int h = blockIdx.x, s = blockIdx.y, tid = threadIdx.x;
  const float* part = a.partial + (int64_t(s) * a.n_q + h) * a.n_split * (D + 2);
  float mloc = -INFINITY;
  for (int i = tid; i < a.n_split; i += NT) mloc = fmaxf(mloc, part[i * (D + 2) + D]);
  red[tid] = mloc;
  __syncthreads();
  for (int o = NT / 2; o > 0; o >>= 1) {
    if (tid < o) red[tid] = fmaxf(red[tid], red[tid + o]);
    __syncthreads();
  }
  const float mmax = red[0];
  __syncthreads();
  float lloc = 0.0f;
  for (int i = tid; i < a.n_split; i += NT) {
    const float mi = part[i * (D + 2) + D];
    const float w = (mi == -INFINITY) ? 0.0f : exp2f(mi - mmax);
    wts[i] = w;
    lloc += w * part[i * (D + 2) + D + 1];
  }
  red[tid] = lloc;
  __syncthreads();
  for (int o = NT / 2; o > 0; o >>= 1) {
    if (tid < o) red[tid] += red[tid + o];
    __syncthreads();
  }
  const float ltot = red[0];
  __syncthreads();
  const int c = tid % D, q = tid / D;
  {
    float v = 0.0f;
#pragma unroll 8
    for (int i = q; i < a.n_split; i += NSUB) v = fmaf(wts[i], part[i * (D + 2) + c], v);
    red[tid] = v;
  }
  __syncthreads();
  if (tid < D) {
    float v = 0.0f;
    for (int qq = 0; qq < NSUB; ++qq) v += red[qq * D + tid];
    accs[tid] = v;
  }
  __syncthreads();
  {
    constexpr int RPER = D / NSUB;
    float v = 0.0f;
#pragma unroll 8
    for (int r = q * RPER; r < (q + 1) * RPER; ++r) v = fmaf(a.rot_v[r * D + c], accs[r], v);
    red[tid] = v;
  }
  __syncthreads();
  if (tid < D) {
    float v = 0.0f;
    for (int qq = 0; qq < NSUB; ++qq) v += red[qq * D + tid];
    const float inv = (ltot > 0.0f) ? 1.0f / (ltot * sqrtf(float(D))) : 0.0f;
    a.out[(int64_t(s) * a.n_q + h) * D + tid] = v * inv;
  }
}

template <int D>
hipError_t launch_decode_d(const DecodeArgs& a, bgtq_dtype q_dt, hipStream_t st) {
  if (q_dt == BGTQ_BF16)
    hipLaunchKernelGGL(k_decode_prep<uint16_t>, dim3(a.n_q, a.batch), dim3(128), 0, st, a);
  else
    hipLaunchKernelGGL(k_decode_prep<float>, dim3(a.n_q, a.batch), dim3(128), 0, st, a);
  const dim3 grid(a.n_split, a.n_kv, a.batch);
  if (a.use_mfma) {
    const int region_words = mfma_region_words(D, 4 * a.chunks + 3, 2 * a.v_bits + 3);
    int nwaves = 4;
    while (nwaves > 1 && (kTableWords + nwaves * region_words) * 4 > 64 * 1024) --nwaves;
    const size_t lds = size_t(kTableWords + nwaves * region_words) * 4;
    hipLaunchKernelGGL(k_decode_mfma<D>, grid, dim3(64 * nwaves), lds, st, a);
  } else {
    const int maxg = a.group <= 1 ? 1 : a.group <= 2 ? 2 : a.group <= 4 ? 4 : a.group <= 8 ? 8 : 16;
    const int RS = 4 * a.chunks + 1, VS = 2 * a.v_bits + 1;
    const int kbuf_words = 64 * RS > D * VS ? 64 * RS : D * VS;
    const int wave_words = kbuf_words + 64 * kMaxGroups + 64 * maxg;
    int nwaves = 4;
    while (nwaves > 1 && (768 + nwaves * wave_words) * 4 > 64 * 1024) --nwaves;
    const size_t lds = size_t(768 + nwaves * wave_words) * 4;
    const dim3 block(64 * nwaves);
    switch (maxg) {
      case 1: hipLaunchKernelGGL((k_decode_split<D, 1>), grid, block, lds, st, a); break;
      case 2: hipLaunchKernelGGL((k_decode_split<D, 2>), grid, block, lds, st, a); break;
      case 4: hipLaunchKernelGGL((k_decode_split<D, 4>), grid, block, lds, st, a); break;
      case 8: hipLaunchKernelGGL((k_decode_split<D, 8>), grid, block, lds, st, a); break;
      default: hipLaunchKernelGGL((k_decode_split<D, 16>), grid, block, lds, st, a); break;
    }
  }
  hipLaunchKernelGGL(k_decode_combine<D>, dim3(a.n_q, a.batch), dim3(1024), 0, st, a);
  return hipGetLastError();
}

}  // namespace

// ===================================================================== launchers

hipError_t upload_tables(const Tables& t) {
  hipError_t e = hipMemcpyToSymbol(HIP_SYMBOL(c_thr), t.thr, sizeof(t.thr));
  if (e == hipSuccess) e = hipMemcpyToSymbol(HIP_SYMBOL(c_cen), t.cen, sizeof(t.cen));
  if (e == hipSuccess) e = hipMemcpyToSymbol(HIP_SYMBOL(c_dgain), t.dgain, sizeof(t.dgain));
  if (e == hipSuccess) e = hipMemcpyToSymbol(HIP_SYMBOL(c_pair), t.pair, sizeof(t.pair));
  if (e == hipSuccess) e = hipMemcpyToSymbol(HIP_SYMBOL(c_single), t.single, sizeof(t.single));
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
                     2 * kHalf * BGTQ_MAX_HEAD_DIM + sizeof(HeadLayout);
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

int decode_splits(int batch, int n_kv_heads, int64_t capacity, bool mfma) {
  const int64_t tiles = capacity / kTile;
  const int64_t units = int64_t(batch) * n_kv_heads;
  int64_t want = (1024 + units - 1) / units;         // about 1024 workgroups in flight
  const int64_t per_split = mfma ? 8 : 8;             // tiles per split at least
  const int64_t by_work = (tiles + per_split - 1) / per_split;
  if (want > by_work) want = by_work;
  if (want < 1) want = 1;
  if (want > 1024) want = 1024;
  return int(want);
}

size_t decode_qrot_bytes(int batch, int n_kv_heads, int d) {
  return size_t(batch) * n_kv_heads * d * kQPad * 4;
}

size_t decode_qmma_bytes(int batch, int n_kv_heads) {
  return size_t(batch) * n_kv_heads * kMaxKSteps * 2 * 64 * 8 * 2;
}

}  // namespace bgtq
