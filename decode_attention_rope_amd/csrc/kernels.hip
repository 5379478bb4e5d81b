// HIP kernels of the Block-GTQ packed-cache decode path, written for gfx950 (CDNA4, wave64).
//
// Method: "RoPE-Aware Bit Allocation for KV-Cache Quantization" (arXiv 2606.24033), abstract.
// Each kernel states the reading of the abstract it implements.  Kernels that must agree
// bit for bit with the specified arithmetic (energy, allocation, quantize-and-pack) are
// compiled without floating-point contraction (-ffp-contract=off) and use only correctly
// rounded fp32/fp64 operations in a fixed order; decode attention uses explicit fmaf.

#include <hip/hip_runtime.h>

#include "bgtq_internal.h"

#include <type_traits>

namespace bgtq {
namespace {

typedef const float __attribute__((address_space(4))) cfloat;
typedef const HeadLayout __attribute__((address_space(4))) cLayout;

__constant__ float c_thr[kMaxBits][255];
__constant__ float c_cen[kMaxBits][256];
__constant__ double c_dgain[kMaxBits];
__constant__ uint32_t c_pair[kPairWords];
__constant__ uint16_t c_single[kSingleHalves];
__constant__ uint2 c_pair_hl[kPairWords];
__constant__ uint32_t c_single_hl[kSingleHalves];

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
// fp16 of a key kept in the recent-key window: nearest-even, saturated at +-65504
__device__ __forceinline__ uint16_t f16_sat_bits(float x) {
  return f32_to_f16_bits(fminf(fmaxf(x, -65504.0f), 65504.0f));
}

// Orders LDS traffic between lanes of one wavefront (all lanes run in lockstep).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// One DPP move of a double (both halves with the same control; lanes without a source, or in
// rows outside row_mask, keep their own value).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ double dpp_f64(double v) {
  const unsigned long long u = __double_as_longlong(v);
  const int lo = int(uint32_t(u)), hi = int(uint32_t(u >> 32));
  const int lo2 = __builtin_amdgcn_update_dpp(lo, lo, CTRL, ROW_MASK, 0xf, false);
  const int hi2 = __builtin_amdgcn_update_dpp(hi, hi, CTRL, ROW_MASK, 0xf, false);
  return __longlong_as_double((long long)((unsigned long long)uint32_t(hi2) << 32 | uint32_t(lo2)));
}
// Maximum of a double over the wavefront, in every lane: a prefix maximum within each row of 16
// lanes (row_shr 1, 2, 4, 8), rows combined by the row broadcasts of lanes 15 and 31, the
// result read from lane 63.
__device__ __forceinline__ double wave_max_f64(double v) {
  v = fmax(v, dpp_f64<0x111, 0xf>(v));
  v = fmax(v, dpp_f64<0x112, 0xf>(v));
  v = fmax(v, dpp_f64<0x114, 0xf>(v));
  v = fmax(v, dpp_f64<0x118, 0xf>(v));
  v = fmax(v, dpp_f64<0x142, 0xa>(v));
  v = fmax(v, dpp_f64<0x143, 0xc>(v));
  const unsigned long long u = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readlane(int(uint32_t(u)), 63), hi = __builtin_amdgcn_readlane(int(uint32_t(u >> 32)), 63);
  return __longlong_as_double((long long)((unsigned long long)uint32_t(hi) << 32 | uint32_t(lo)));
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
  const uint32_t h = uint32_t(m) / 2u - 1u;             // number of smaller sizes
  return size_t(4u * (h * (h + 1u) * (2u * h + 1u) / 6u));   // m <= 256: fits 32 bits
}

// Layers per size the kernels apply; the records' header must not name more.
constexpr int kMaxGivensLayers = 16;

// Structured (Givens-layer) rotations: header row m/2 - 1 = (first record row of size m,
// layer count); record (a | b << 16, cos, sin) of pair slot i of layer l of size m at row
// first + l * m/2 + i.  One pair rotation in place: y_a = c x_a - s x_b, y_b = s x_a + c x_b,
// every product and sum rounded (this file is compiled without contraction).
__device__ __forceinline__ void givens_pair(float* x, uint4 rec) {
  const int ia = int(rec.x & 0xffffu), ib = int(rec.x >> 16);
  const float c = __uint_as_float(rec.y), s = __uint_as_float(rec.z);
  const float xa = x[ia], xb = x[ib];
  x[ia] = c * xa - s * xb;
  x[ib] = s * xa + c * xb;
}
// record of pair slot q (storage positions 2q, 2q + 1 lie in one width group) in layer l, or
// a zero record when the group's size has fewer layers
__device__ __forceinline__ bool givens_slot(const uint4* G, const HeadLayout& L, int q, int l, uint4& rec, int& first) {
  const int g = L.group[2 * q], m = L.g_m[g];
  first = L.g_first[g];
  const uint4 h = G[m / 2 - 1];
  if (l >= min(int(h.y), kMaxGivensLayers)) return false;
  rec = G[h.x + l * (m / 2) + (q - first / 2)];
  return true;
}
__device__ __forceinline__ int givens_count(const uint4* G, int m) { return min(int(G[m / 2 - 1].y), kMaxGivensLayers); }
// most layers among a layout's width groups
__device__ __forceinline__ int givens_layers(const uint4* G, const HeadLayout& L) {
  int n = 0;
  for (int g = 0; g < L.n_groups; ++g) n = max(n, givens_count(G, L.g_m[g]));
  return n;
}
// One thread's pair slot through the layers of size m: the records of the next kGivensAhead
// layers are kept in registers and refilled as layers are applied, so the layers run without
// waiting on memory.  Every index is a compile-time constant once the layer loop is unrolled.
constexpr int kGivensAhead = 8;
struct GivensSlot {
  uint32_t ab[kGivensAhead];
  float c[kGivensAhead], s[kGivensAhead];
  const uint4* rec;    // record of layer 0; layer l at rec[l * stride]
  int stride, n;
  __device__ __forceinline__ void fetch(int l) {
    if (l < n) {
      const uint4 r = rec[l * stride];
      ab[l % kGivensAhead] = r.x;
      c[l % kGivensAhead] = __uint_as_float(r.y);
      s[l % kGivensAhead] = __uint_as_float(r.z);
    }
  }
  // layer l on x (forward, exact rounding sequence); then the record kGivensAhead layers on
  __device__ __forceinline__ void apply(float* x, int l) {
    const int k = l % kGivensAhead, ia = int(ab[k] & 0xffffu), ib = int(ab[k] >> 16);
    const float xa = x[ia], xb = x[ib];
    x[ia] = c[k] * xa - s[k] * xb;
    x[ib] = s[k] * xa + c[k] * xb;
  }
};
__device__ __forceinline__ void givens_fetch(const uint4* G, int m, int slot, GivensSlot& g) {
  const uint4 h = G[m / 2 - 1];
  g.n = min(int(h.y), kMaxGivensLayers);
  g.rec = G + h.x + slot;
  g.stride = m / 2;
#pragma unroll
  for (int l = 0; l < kGivensAhead; ++l) g.fetch(l);
}

// ===================================================================== block energy
// Label-free energy of RoPE block j (abstract: one score per RoPE block, per layer and KV
// head, no labels needed).  Reading: mean over tokens of the squared norm of the block's
// two coordinates, fp64, summed in ascending t within 256-token chunks, chunks in
// ascending order.  Pass 1: one thread per (head, chunk, block); lanes run over blocks
// so every token row is read coalesced.  Pass 2: one thread per (head, block).
template <typename T>
__global__ __launch_bounds__(256) void k_energy_partial(const T* __restrict__ keys, int n_heads, int64_t n_tokens, int n,
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
  int64_t t = t0;
  // 16 tokens' loads are requested before their adds, which keep ascending token order
  for (; t + 16 <= t1; t += 16) {
    float xa[16], xb[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      xa[i] = load_f(base, (t + i) * st + ca);
      xb[i] = load_f(base, (t + i) * st + cb);
    }
    __builtin_amdgcn_sched_barrier(0);     // every load issued before the first add
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const double x0 = (double)xa[i], x1 = (double)xb[i];
      const double e = x0 * x0 + x1 * x1;
      acc = acc + e;
    }
  }
  for (; t < t1; ++t) {
    const double x0 = (double)load_f(base, t * st + ca);
    const double x1 = (double)load_f(base, t * st + cb);
    const double e = x0 * x0 + x1 * x1;
    acc = acc + e;
  }
  part[(int64_t(h) * n_chunks + c) * n + j] = acc;
}

// Sum of a block's chunk partials in ascending chunk order (p: the block's first partial,
// consecutive chunks n apart); B loads are requested before their adds.
template <int B>
__device__ __forceinline__ double chunk_sum(const double* __restrict__ p, int n_chunks, int n) {
  double tot = 0.0;
  int c = 0;
  for (; c + B <= n_chunks; c += B) {
    double v[B];
#pragma unroll
    for (int i = 0; i < B; ++i) v[i] = p[int64_t(c + i) * n];
    __builtin_amdgcn_sched_barrier(0);     // every load issued before the first add
#pragma unroll
    for (int i = 0; i < B; ++i) tot = tot + v[i];
  }
  for (; c < n_chunks; ++c) tot = tot + p[int64_t(c) * n];
  return tot;
}

__global__ void k_energy_final(const double* __restrict__ part, int n_heads, int n_chunks, int n,
                               int64_t n_tokens, double* __restrict__ out) {
  const int gid = blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= n_heads * n) return;
  const int h = gid / n, j = gid % n;
  out[gid] = chunk_sum<8>(part + int64_t(h) * n_chunks * n + j, n_chunks, n) / (double)n_tokens;
}

// ===================================================================== greedy allocation
// Integer widths by marginal gain (abstract: greedy, integer widths, more bits where the
// energy is high, matched budget).  Reading: every block starts at b_min; each of the
// `increments` steps gives one bit to the block of largest fp64 gain E_j*(D(b_j)-D(b_j+1))
// among blocks below b_max, ties to the lowest j.  One wavefront per head, block j on
// lane j % 64; each step takes the wave's largest gain, then the lowest block index at it.
// The width groups and the K record layout follow from the number of blocks per width.
// One wavefront allocates one head from its energies e0 (block lane) and e1 (block lane + 64)
// and writes the widths and the layout descriptor.
__device__ __forceinline__ void allocate_wave(double e0, double e1, int n, int increments, int b_min, int b_max,
                                              int pairing, uint8_t* __restrict__ widths_h,
                                              HeadLayout* __restrict__ layout_h) {
  __shared__ HeadLayout lay;
  __shared__ double dg[kMaxBits];          // D(b) - D(b + 1)
  const int lane = threadIdx.x;
  const int j0 = lane, j1 = lane + 64;
  if (lane < kMaxBits) dg[lane] = c_dgain[lane];
  __syncthreads();
  auto gain = [&](double e, int w) { return e * dg[w]; };   // w < kMaxBits
  int w0 = b_min, w1 = b_min;
  for (int it = 0; it < increments; ++it) {
    const double g0 = (j0 < n && w0 < b_max) ? gain(e0, w0) : -1.0;
    const double g1 = (j1 < n && w1 < b_max) ? gain(e1, w1) : -1.0;
    const bool up = g1 > g0;               // the lane's better block (j0 on a tie)
    const double g = up ? g1 : g0;
    const double gm = wave_max_f64(g);
    // the lowest block index among the lanes at the maximum: blocks j0 < 64 <= j1
    const unsigned long long m_lo = __ballot(g == gm && !up), m_hi = __ballot(g == gm && up);
    const int win = m_lo ? __ffsll(m_lo) - 1 : 64 + __ffsll(m_hi) - 1;
    if (win == j0) ++w0;
    else if (win == j1) ++w1;
  }
  if (j0 < n) widths_h[j0] = uint8_t(w0);
  if (j1 < n) widths_h[j1] = uint8_t(w1);
  uint32_t* lw = reinterpret_cast<uint32_t*>(&lay);
  for (int i = lane; i < int(sizeof(HeadLayout) / 4); i += 64) lw[i] = 0;
  // Width groups in descending width, blocks of one width in ascending index: from the
  // blocks per width, each group's first storage position and record bit, and each block's
  // rank within its width.
  unsigned long long mk0[kMaxBits + 1], mk1[kMaxBits + 1];
  int cnt[kMaxBits + 1], gidx[kMaxBits + 1], fpos[kMaxBits + 1], fbit[kMaxBits + 1];
#pragma unroll
  for (int w = 1; w <= kMaxBits; ++w) {
    mk0[w] = __ballot(j0 < n && w0 == w);
    mk1[w] = __ballot(j1 < n && w1 == w);
    cnt[w] = __popcll(mk0[w]) + __popcll(mk1[w]);
  }
  int ng = 0, pos = 0, bit = 0;
#pragma unroll
  for (int w = kMaxBits; w >= 1; --w) {
    gidx[w] = ng;
    fpos[w] = pos;
    fbit[w] = bit;
    if (cnt[w] > 0) ++ng;
    pos += 2 * cnt[w];
    bit += 2 * w * cnt[w];
  }
  __syncthreads();
  if (lane == 0) {
#pragma unroll
    for (int w = kMaxBits; w >= 1; --w) {
      if (cnt[w] > 0) {
        const int g = gidx[w];
        lay.g_width[g] = w; lay.g_first[g] = fpos[w]; lay.g_m[g] = 2 * cnt[w]; lay.g_bitoff[g] = fbit[w];
      }
    }
    lay.n_groups = ng; lay.d_eff = pos; lay.code_bits = bit; lay.chunks = (bit + 127) / 128;
  }
  const unsigned long long below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  auto place = [&](int j, int w, int rank) {     // block j (width w >= 1) at its rank among width w
    int g = 0, p = 0, b = 0;
#pragma unroll
    for (int ww = 1; ww <= kMaxBits; ++ww)
      if (w == ww) { g = gidx[ww]; p = fpos[ww]; b = fbit[ww]; }
    p += 2 * rank;
    b += 2 * w * rank;
    const int ca = pairing ? 2 * j : j, cb = pairing ? 2 * j + 1 : j + n;
    lay.perm[p] = uint8_t(ca); lay.group[p] = uint8_t(g); lay.offset[p] = uint16_t(b);
    lay.perm[p + 1] = uint8_t(cb); lay.group[p + 1] = uint8_t(g); lay.offset[p + 1] = uint16_t(b + w);
  };
  {
    unsigned long long s0 = 0, a0 = 0, s1 = 0;
#pragma unroll
    for (int w = 1; w <= kMaxBits; ++w) {
      if (w0 == w) s0 = mk0[w];
      if (w1 == w) { a0 = mk0[w]; s1 = mk1[w]; }
    }
    if (j0 < n && w0 >= 1) place(j0, w0, __popcll(s0 & below));
    if (j1 < n && w1 >= 1) place(j1, w1, __popcll(a0) + __popcll(s1 & below));
  }
  // storage positions with bits in record dword `lane`: each group holds positions at bits
  // bitoff + i * w, so the counts below a bit are closed forms per group
  if (lane < 4 * ((bit + 127) / 128)) {
    const int b_lo = 32 * lane, b_hi = b_lo + 32;
    int first = 0, end = 0;
#pragma unroll
    for (int w = 1; w <= kMaxBits; ++w) {
      const int m = 2 * cnt[w], bo = fbit[w];
      const int c_end = b_hi > bo ? (b_hi - bo + w - 1) / w : 0;     // positions starting below b_hi
      const int c_first = b_lo >= bo ? (b_lo - bo) / w : 0;          // positions ending at or below b_lo
      end += c_end < m ? c_end : m;
      first += c_first < m ? c_first : m;
    }
    lay.dw_first[lane] = uint16_t(first);
    lay.dw_end[lane] = uint16_t(end);
  }
  __syncthreads();
  if (lane == 0) {
    // matrix-core view: segments of at most 8 positions in storage order; a k-step takes up to
    // 4 consecutive segments from at most two groups (the two halves of the output columns)
    int ks = -1, slot = 4, ga = -1, gb = -1;
    for (int gg = 0; gg < ng; ++gg) {
      const int w = lay.g_width[gg], m = lay.g_m[gg], first = lay.g_first[gg], bo = lay.g_bitoff[gg];
      for (int s0 = 0; s0 < m; s0 += kSegLen) {
        if (slot == 4 || (gg != ga && gg != gb && gb >= 0)) {
          if (ks >= 0) lay.kgroups[ks] = uint32_t(ga) | uint32_t(gb >= 0 ? gb : ga) << 8;
          ++ks; slot = 0; ga = gg; gb = -1;
        } else if (gg != ga && gb < 0) {
          gb = gg;
        }
        const int cnt_s = m - s0 < kSegLen ? m - s0 : kSegLen;
        const uint32_t half = gg == ga ? 0u : 1u;
        lay.seg[4 * ks + slot] = uint32_t(bo + s0 * w) | uint32_t(w) << 16 | uint32_t(gg) << 20 |
                                 uint32_t(cnt_s) << 24 | half << 28;
        for (int e = 0; e < cnt_s; ++e) lay.kpos[first + s0 + e] = uint16_t(32 * ks + kSegLen * slot + e);
        ++slot;
      }
    }
    if (ks >= 0) lay.kgroups[ks] = uint32_t(ga) | uint32_t(gb >= 0 ? gb : ga) << 8;
    lay.n_ksteps = ks + 1;
    for (int i = 0; i < 4 * lay.n_ksteps; ++i)
      if (lay.seg[i] == 0u) lay.seg[i] = 1u << 16;   // unused slot: width 1 at bit 0
  }
  __syncthreads();
  uint32_t* dst = reinterpret_cast<uint32_t*>(layout_h);
  for (int i = lane; i < int(sizeof(HeadLayout) / 4); i += 64) dst[i] = lw[i];
}

__global__ __launch_bounds__(64) void k_allocate(const double* __restrict__ energy, int n, int increments,
                                                 int b_min, int b_max, int pairing,
                                                 uint8_t* __restrict__ widths,
                                                 HeadLayout* __restrict__ layouts) {
  const int h = blockIdx.x, lane = threadIdx.x;
  const double e0 = lane < n ? energy[int64_t(h) * n + lane] : 0.0;
  const double e1 = lane + 64 < n ? energy[int64_t(h) * n + lane + 64] : 0.0;
  allocate_wave(e0, e1, n, increments, b_min, b_max, pairing, widths + int64_t(h) * n, layouts + h);
}

// Prefill: the energy's final reduction and the allocation of one head in one wavefront
// (the same sums in the same order as k_energy_final, then k_allocate's arithmetic).
__global__ __launch_bounds__(64) void k_energy_allocate(const double* __restrict__ part, int n_chunks,
                                                        int64_t n_tokens, int n, int increments, int b_min,
                                                        int b_max, int pairing, double* __restrict__ energy_out,
                                                        uint8_t* __restrict__ widths, HeadLayout* __restrict__ layouts) {
  const int h = blockIdx.x, lane = threadIdx.x;
  const double* p = part + int64_t(h) * n_chunks * n;
  const double e0 = lane < n ? chunk_sum<32>(p + lane, n_chunks, n) / (double)n_tokens : 0.0;
  const double e1 = lane + 64 < n ? chunk_sum<32>(p + lane + 64, n_chunks, n) / (double)n_tokens : 0.0;
  if (energy_out) {
    if (lane < n) energy_out[int64_t(h) * n + lane] = e0;
    if (lane + 64 < n) energy_out[int64_t(h) * n + lane + 64] = e1;
  }
  allocate_wave(e0, e1, n, increments, b_min, b_max, pairing, widths + int64_t(h) * n, layouts + h);
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

// Slot geometry of k_append: each of the four waves owns 8 of the workgroup's 32 slots, and
// everything per slot (norms, rotations, codes) runs inside the owning wave, ordered by
// wave_sync() alone.  Keys or values of the 32 slots sit in LDS coordinate-major,
// xt[c * kXTS + r] (row stride 36 floats, 16-byte aligned), so one coordinate of a wave's 8
// slots is two 16-byte reads.
constexpr int kWaveSlots = 8;
constexpr int kXTS = kHalf + 4;

// Sequential fp32 dot products of two matrix rows (o, o + 1 of an m x m matrix stored
// transposed: element (o, k) at rt[k * ld], (o + 1, k) next to it) with the coordinates of 8
// slots, x[k * kXTS + j]: k ascending from 0, every product and sum rounded.  The matrix pairs
// are requested 8 k-steps ahead of their use.
__device__ __forceinline__ void dot_pair8(const float* __restrict__ rt, int ld, int m, const float* x,
                                          float (&acc)[2][kWaveSlots]) {
  constexpr int KB = 8;
  float2 rc[KB];
#pragma unroll
  for (int i = 0; i < KB; ++i)
    rc[i] = i < m ? *reinterpret_cast<const float2*>(rt + size_t(i) * ld) : make_float2(0.0f, 0.0f);
  for (int k0 = 0; k0 < m; k0 += KB) {
    float2 rn[KB];
#pragma unroll
    for (int i = 0; i < KB; ++i)
      rn[i] = k0 + KB + i < m ? *reinterpret_cast<const float2*>(rt + size_t(k0 + KB + i) * ld)
                              : make_float2(0.0f, 0.0f);
#pragma unroll
    for (int i = 0; i < KB; ++i) {
      if (k0 + i < m) {
        const float4* x4 = reinterpret_cast<const float4*>(x + (k0 + i) * kXTS);
        const float4 xa = x4[0], xb = x4[1];
        const float xv[kWaveSlots] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
#pragma unroll
        for (int j = 0; j < kWaveSlots; ++j) {
          acc[0][j] = acc[0][j] + rc[i].x * xv[j];
          acc[1][j] = acc[1][j] + rc[i].y * xv[j];
        }
      }
    }
#pragma unroll
    for (int i = 0; i < KB; ++i) rc[i] = rn[i];
  }
}

// One structured-rotation layer of a pair slot on 8 slots: x points at coordinate 0 of the
// slot's width group (coordinate-major, stride kXTS); same rounding as GivensSlot::apply.
__device__ __forceinline__ void givens_apply8(float* x, const GivensSlot& gs, int l) {
  const int k = l % kGivensAhead, ia = int(gs.ab[k] & 0xffffu), ib = int(gs.ab[k] >> 16);
  const float c = gs.c[k], sn = gs.s[k];
  float4* pa = reinterpret_cast<float4*>(x + ia * kXTS);
  float4* pb = reinterpret_cast<float4*>(x + ib * kXTS);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const float4 xa = pa[h], xb = pb[h];
    float4 ya, yb;
    ya.x = c * xa.x - sn * xb.x; yb.x = sn * xa.x + c * xb.x;
    ya.y = c * xa.y - sn * xb.y; yb.y = sn * xa.y + c * xb.y;
    ya.z = c * xa.z - sn * xb.z; yb.z = sn * xa.z + c * xb.z;
    ya.w = c * xa.w - sn * xb.w; yb.w = sn * xa.w + c * xb.w;
    pa[h] = ya;
    pb[h] = yb;
  }
}

// Sequential fp32 sum of squares of m coordinates of one slot (x[k * kXTS], k ascending).
__device__ __forceinline__ float sum_sq_slot(const float* x, int m) {
  float ss = 0.0f;
  int k = 0;
  for (; k + 8 <= m; k += 8) {
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = x[(k + i) * kXTS];
#pragma unroll
    for (int i = 0; i < 8; ++i) ss = ss + v[i] * v[i];
  }
  for (; k < m; ++k) ss = ss + x[k * kXTS] * x[k * kXTS];
  return ss;
}

// LDS of k_append for head dim d (at most DM): the slot tile, thresholds, norms, key and value
// codes, layout descriptor.
__host__ __device__ constexpr size_t append_lds_bytes(int d, int dm) {
  return size_t(d) * kXTS * 4 + kMaxBits * 255 * 4 + kHalf * kMaxGroups * 4 + kHalf * 4 + 2 * size_t(kHalf) * dm +
         sizeof(HeadLayout);
}

// Codes of a wave's 8 slots at one storage position or coordinate: z = (y / n) * fl32(sqrt(m)),
// code = number of thresholds below z (0 for a zero norm).  The 8 binary searches advance
// together, so each step's threshold reads are independent of one another.
__device__ __forceinline__ void codes8(const float* y, const float* nrm, int nstride, const float* thr, int bits,
                                       float sq, int rw, int ra, int rb, uint8_t* dst, int dstride) {
  float z[kWaveSlots];
  bool zero[kWaveSlots];
  int code[kWaveSlots];
#pragma unroll
  for (int j = 0; j < kWaveSlots; ++j) {
    const float nv = nrm[(rw + j) * nstride];
    zero[j] = nv == 0.0f;
    z[j] = (y[j] / nv) * sq;
    code[j] = 0;
  }
  for (int b = bits - 1; b >= 0; --b) {
#pragma unroll
    for (int j = 0; j < kWaveSlots; ++j) {
      const int cand = code[j] | (1 << b);
      if (z[j] > thr[cand - 1]) code[j] = cand;
    }
  }
#pragma unroll
  for (int j = 0; j < kWaveSlots; ++j) {
    const int r = rw + j;
    if (r >= ra && r < rb) dst[r * dstride] = uint8_t(zero[j] ? 0 : code[j]);
  }
}

template <typename T, int DM, bool GIV>
__global__ __launch_bounds__(256) void k_append(AppendArgs a) {
  extern __shared__ __align__(16) float sm[];
  constexpr int QL = (DM / 2 + 63) / 64;           // pair slots per lane
  constexpr int PL = DM / 64;                      // coordinates per lane
  const int d = a.d;
  const int si = blockIdx.z, s = a.seq_begin + si, hk = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t len = a.lengths[s];
  if (len + a.n_new > a.capacity) {
    if (blockIdx.x == 0 && hk == 0 && tid == 0 && a.status) atomicOr(a.status, 1);
    return;
  }
  const int64_t ht = len / kHalf + blockIdx.x;
  const int64_t lo = len > ht * kHalf ? len : ht * kHalf;
  const int64_t hi = (len + a.n_new) < (ht + 1) * kHalf ? (len + a.n_new) : (ht + 1) * kHalf;
  if (lo >= hi) return;
  const int r0 = int(lo - ht * kHalf), r1 = int(hi - ht * kHalf);   // appended slots r0 .. r1 - 1
  const int64_t tile = ht / 2;
  const int half = int(ht & 1);
  float* xt = sm;                                   // [d][kXTS] keys (storage order), then values
  float* thr = xt + d * kXTS;                       // [8][255]
  float* knrm = thr + kMaxBits * 255;               // [32][8]
  float* vnrm = knrm + kHalf * kMaxGroups;          // [32]
  uint8_t* kcode = reinterpret_cast<uint8_t*>(vnrm + kHalf);   // [32][DM]
  uint8_t* vcode = kcode + kHalf * DM;                          // [32][DM]
  HeadLayout* Ls = reinterpret_cast<HeadLayout*>(vcode + kHalf * DM);

  static_assert(BGTQ_LAYOUT_BYTES == 256 * 16, "one 16-byte piece of the layout per thread");
  reinterpret_cast<uint4*>(Ls)[tid] = reinterpret_cast<const uint4*>(a.layouts + int64_t(s) * a.n_kv_heads + hk)[tid];
  for (int i = tid; i < kMaxBits * 255; i += 256) thr[i] = c_thr[i / 255][i % 255];
  __syncthreads();
  const HeadLayout& L = *Ls;
  const int ng = L.n_groups, d_eff = L.d_eff, n_dw = 4 * a.chunks;
  const size_t reg = size_t(s) * a.n_kv_heads + hk;
  const int64_t tiles = a.capacity / kTile;
  const T* kin = static_cast<const T*>(a.keys) + si * a.stride_seq + hk * a.stride_head;
  const T* vin = static_cast<const T*>(a.values) + si * a.stride_seq + hk * a.stride_head;
  const int64_t tok0 = ht * kHalf - len;            // input token of slot 0
  const int rw = kWaveSlots * wave;                 // this wave's slots rw .. rw + 7
  const int ra = max(r0, rw), rb = min(r1, rw + kWaveSlots);   // of which appended: ra .. rb - 1
  const bool busy = ra < rb;
  float* const xw = xt + rw;                        // this wave's column of the slot tile

  // ---- keys, in the owning wave: load (storage order; slots not appended hold zeros), group
  // norms, rotation, codes
  if (busy) {
    float kv[kWaveSlots][PL];
#pragma unroll
    for (int j = 0; j < kWaveSlots; ++j) {
      const int r = rw + j;
#pragma unroll
      for (int i = 0; i < PL; ++i) {
        const int p = lane + 64 * i;
        kv[j][i] = (r >= ra && r < rb && p < d_eff) ? load_f(kin, (tok0 + r) * a.stride_token + L.perm[p]) : 0.0f;
      }
    }
    __builtin_amdgcn_sched_barrier(0);     // every load issued before the first store
#pragma unroll
    for (int j = 0; j < kWaveSlots; ++j) {
#pragma unroll
      for (int i = 0; i < PL; ++i) {
        const int p = lane + 64 * i;
        if (p < d_eff) xw[p * kXTS + j] = kv[j][i];
      }
    }
    wave_sync();
    {
      const int j = lane & 7, g = lane >> 3, r = rw + j;
      if (g < ng && r >= ra && r < rb) knrm[r * kMaxGroups + g] = sqrtf(sum_sq_slot(xw + L.g_first[g] * kXTS + j, L.g_m[g]));
    }
    wave_sync();
    if constexpr (GIV) {
      const uint4* const giv = a.givens;
      GivensSlot gs[QL];
      int first[QL];
#pragma unroll
      for (int i = 0; i < QL; ++i) {
        const int q = lane + 64 * i;
        gs[i].n = 0;
        first[i] = 0;
        if (q < d_eff / 2) {
          const int g = L.group[2 * q];
          first[i] = L.g_first[g];
          givens_fetch(giv, L.g_m[g], q - first[i] / 2, gs[i]);
        }
      }
      const int nl = givens_layers(giv, L);
#pragma unroll
      for (int l = 0; l < kMaxGivensLayers; ++l) {
        if (l < nl) {
#pragma unroll
          for (int i = 0; i < QL; ++i) {
            if (l < gs[i].n) {
              givens_apply8(xw + first[i] * kXTS, gs[i], l);
              if (l + kGivensAhead < kMaxGivensLayers) gs[i].fetch(l + kGivensAhead);
            }
          }
          wave_sync();
        }
      }
#pragma unroll
      for (int i = 0; i < PL; ++i) {
        const int p = lane + 64 * i;
        if (p < d_eff) {
          const int g = L.group[p], w = L.g_width[g];
          const float4* x4 = reinterpret_cast<const float4*>(xw + p * kXTS);
          const float4 xa = x4[0], xb = x4[1];
          const float y[kWaveSlots] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
          codes8(y, knrm + g, kMaxGroups, thr + (w - 1) * 255, w, sqrtf(float(L.g_m[g])), rw, ra, rb, kcode + p, DM);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < QL; ++i) {
        const int q = lane + 64 * i;
        if (q < d_eff / 2) {
          const int p = 2 * q, g = L.group[p], m = L.g_m[g], first = L.g_first[g], w = L.g_width[g];
          float acc[2][kWaveSlots] = {};
          dot_pair8(a.rot_bank_t + bank_offset(m) + (p - first), m, m, xw + first * kXTS, acc);
          const float sq = sqrtf(float(m));
          codes8(acc[0], knrm + g, kMaxGroups, thr + (w - 1) * 255, w, sq, rw, ra, rb, kcode + p, DM);
          codes8(acc[1], knrm + g, kMaxGroups, thr + (w - 1) * 255, w, sq, rw, ra, rb, kcode + p + 1, DM);
        }
      }
    }
  }
  __syncthreads();

  // ---- values, in the owning wave (loads requested before the key records are packed)
  float vv[kWaveSlots][PL];
  if (busy) {
#pragma unroll
    for (int j = 0; j < kWaveSlots; ++j) {
      const int r = rw + j;
#pragma unroll
      for (int i = 0; i < PL; ++i) {
        const int c = lane + 64 * i;
        vv[j][i] = (r >= ra && r < rb && c < d) ? load_f(vin, (tok0 + r) * a.stride_token + c) : 0.0f;
      }
    }
  }
  // pack key records (one thread per (slot, record dword)) and key norms
  uint32_t* kc = reinterpret_cast<uint32_t*>(a.k_codes) + reg * tiles * a.chunks * kTile * 4;
  const int nrows = r1 - r0;
  for (int it = tid; it < nrows * n_dw; it += 256) {
    const int r = r0 + it % nrows, w = it / nrows;
    const int64_t slot = ht * kHalf + r;
    uint32_t v = 0;
    for (int p = L.dw_first[w]; p < L.dw_end[w]; ++p) {
      const uint32_t c = kcode[r * DM + p];
      const int o = int(L.offset[p]) - 32 * w;
      v |= o >= 0 ? (c << o) : (c >> (-o));
    }
    kc[((tile * a.chunks + w / 4) * kTile + (slot % kTile)) * 4 + (w % 4)] = v;
  }
  uint16_t* kn = a.k_norms + reg * tiles * kMaxGroups * kTile;
  for (int it = tid; it < nrows * ng; it += 256) {
    const int r = r0 + it % nrows, g = it / nrows;
    const int64_t slot = ht * kHalf + r;
    kn[(tile * kMaxGroups + g) * kTile + slot % kTile] = f32_to_f16_bits(fminf(knrm[r * kMaxGroups + g], 65504.0f));
  }
  if (busy) {
#pragma unroll
    for (int j = 0; j < kWaveSlots; ++j) {
#pragma unroll
      for (int i = 0; i < PL; ++i) {
        const int c = lane + 64 * i;
        if (c < d) xw[c * kXTS + j] = vv[j][i];
      }
    }
    wave_sync();
    if (lane < kWaveSlots) {
      const int r = rw + lane;
      if (r >= ra && r < rb) vnrm[r] = sqrtf(sum_sq_slot(xw + lane, d));
    }
    wave_sync();
    const int bv = a.v_bits;
    const float sd = sqrtf(float(d));
    if constexpr (GIV) {
      const uint4* const giv = a.givens;
      GivensSlot gs[QL];
#pragma unroll
      for (int i = 0; i < QL; ++i) {
        const int q = lane + 64 * i;
        gs[i].n = 0;
        if (q < d / 2) givens_fetch(giv, d, q, gs[i]);
      }
      const int nl = givens_count(giv, d);
#pragma unroll
      for (int l = 0; l < kMaxGivensLayers; ++l) {
        if (l < nl) {
#pragma unroll
          for (int i = 0; i < QL; ++i) {
            if (l < gs[i].n) {
              givens_apply8(xw, gs[i], l);
              if (l + kGivensAhead < kMaxGivensLayers) gs[i].fetch(l + kGivensAhead);
            }
          }
          wave_sync();
        }
      }
#pragma unroll
      for (int i = 0; i < PL; ++i) {
        const int c = lane + 64 * i;
        if (c < d) {
          const float4* x4 = reinterpret_cast<const float4*>(xw + c * kXTS);
          const float4 xa = x4[0], xb = x4[1];
          const float y[kWaveSlots] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
          codes8(y, vnrm, 1, thr + (bv - 1) * 255, bv, sd, rw, ra, rb, vcode + c, DM);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < QL; ++i) {
        const int q = lane + 64 * i;
        if (q < d / 2) {
          float acc[2][kWaveSlots] = {};
          dot_pair8(a.rot_v_t + 2 * q, d, d, xw, acc);
          codes8(acc[0], vnrm, 1, thr + (bv - 1) * 255, bv, sd, rw, ra, rb, vcode + 2 * q, DM);
          codes8(acc[1], vnrm, 1, thr + (bv - 1) * 255, bv, sd, rw, ra, rb, vcode + 2 * q + 1, DM);
        }
      }
    }
  }
  __syncthreads();
  // pack value segments (one thread per (coordinate, segment dword) of this half tile)
  const int bv = a.v_bits;
  uint32_t* vc = reinterpret_cast<uint32_t*>(a.v_codes) + reg * tiles * d * 2 * bv;
  const uint32_t vmask = (1u << bv) - 1u;
  for (int it = tid; it < d * bv; it += 256) {
    const int i = it / bv, w = half * bv + it % bv;
    uint32_t* addr = vc + (size_t(tile) * d + i) * 2 * bv + w;
    const int bit0 = 32 * w;
    const int j_lo = bit0 / bv, j_hi = (bit0 + 31) / bv;
    // only dwords that hold bits of an appended slot are rewritten; one whose every slot is
    // appended is not read first
    if (tile * kTile + j_hi < lo || tile * kTile + j_lo >= hi) continue;
    const bool whole = tile * kTile + j_lo >= lo && tile * kTile + j_hi < hi;
    uint32_t v = whole ? 0u : *addr;
    for (int j = j_lo; j <= j_hi; ++j) {
      const int64_t slot = tile * kTile + j;
      if (slot < lo || slot >= hi) continue;
      const uint32_t c = vcode[int(slot - ht * kHalf) * DM + i];
      const int o = j * bv - bit0;
      if (o >= 0) v = (v & ~(vmask << o)) | (c << o);
      else v = (v & ~(vmask >> (-o))) | (c >> (-o));
    }
    *addr = v;
  }
  uint16_t* vn = a.v_norms + reg * tiles * kTile;
  for (int r = r0 + tid; r < r1; r += 256) {
    const int64_t slot = ht * kHalf + r;
    vn[tile * kTile + slot % kTile] = f32_to_f16_bits(fminf(vnrm[r], 65504.0f));
  }
}

// Decode-time append of one token to each sequence (n_new == 1), same arithmetic as
// k_append.  One workgroup of 1024 threads per (sequence, KV head): threads 0..d-1 rotate the
// value, d..d+d_eff-1 the key positions, 768.. form the norms.  Reads come in two rounds: first
// everything that depends neither on the sequence length nor on the layout (layout, key, value,
// quantizer thresholds and, for head_dim <= 128, the value rotation), then the slot's old value
// dwords and, with dense rotations and head_dim <= 128, the key groups' matrices.  Both
// rotations are staged in LDS with rows padded to m + 1 floats, so lanes on consecutive rows hit
// distinct banks.  The sequence length is advanced afterwards (k_advance).
//
// Sequential fp32 dot product of row `row` of an m x m matrix stored transposed (element
// (row, k) at Rt[k * m + row]) with x, k ascending, no fused multiply-add; lanes on
// consecutive rows read consecutive floats.  The loop runs to mu >= m (the same bound for
// the whole wavefront, rounded up to 16, read from x): terms with k >= m are exact zeros and
// leave the sum unchanged.  Up to 32 terms are requested before the first add.  x is 8-byte
// aligned.
__device__ __forceinline__ float dot_rows_t(const float* __restrict__ Rt, int m, int mu, int row, const float* x) {
  float acc = 0.0f;
  for (int k0 = 0; k0 < mu; k0 += 32) {
    float r[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const int k = k0 + i < m ? k0 + i : m - 1;
      if (i < 16 || k0 + i < mu) r[i] = Rt[size_t(k) * m + row];
    }
#pragma unroll
    for (int b = 0; b < 32; b += 16) {
      if (b == 0 || k0 + b < mu) {
        float xv[16];
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
          const float2 v = *reinterpret_cast<const float2*>(x + k0 + b + i);
          xv[i] = v.x; xv[i + 1] = v.y;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const bool in = k0 + b + i < m;
          acc = acc + (in ? r[b + i] : 0.0f) * (in ? xv[i] : 0.0f);
        }
      }
    }
  }
  return acc;
}

// Sequential fp32 dot product of row `row` of an LDS matrix with row stride ld and x (both in
// LDS), k ascending over [0, m).  Chunks of 16 terms; each chunk's reads are issued before the
// previous chunk's adds.  Terms past m in the last chunk are exact zeros, which leave the sum's
// value (and so every code) unchanged.  x is 8-byte aligned and readable to the end of that
// chunk.
__device__ __forceinline__ float dot_rows_lds_any(const float* R, int ld, int m, int row, const float* x) {
  const float* rr = R + row * ld;
  float acc = 0.0f;
  float r[16], xv[16];
  auto fetch = [&](float (&rb)[16], float (&xb)[16], int k0) {
#pragma unroll
    for (int i = 0; i < 16; ++i) rb[i] = rr[k0 + i < m ? k0 + i : m - 1];
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
      const float2 v = *reinterpret_cast<const float2*>(x + k0 + i);
      xb[i] = v.x; xb[i + 1] = v.y;
    }
  };
  fetch(r, xv, 0);
  int k0 = 0;
  for (; k0 + 16 < m; k0 += 16) {           // full chunks with a chunk after them
    float rn[16], xn[16];
    fetch(rn, xn, k0 + 16);
#pragma unroll
    for (int i = 0; i < 16; ++i) acc = acc + r[i] * xv[i];
#pragma unroll
    for (int i = 0; i < 16; ++i) { r[i] = rn[i]; xv[i] = xn[i]; }
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {            // the last chunk
    const bool in = k0 + i < m;
    acc = acc + (in ? r[i] : 0.0f) * (in ? xv[i] : 0.0f);
  }
  return acc;
}

// Sequential fp32 sum of squares of x[0..m) (m even, x 8-byte aligned, readable to the end of
// the last chunk of 8); each chunk's reads are issued before the previous chunk's adds.
__device__ __forceinline__ float seq_sumsq(const float* x, int m) {
  float ss = 0.0f;
  float v[8];
  auto fetch = [&](float (&b)[8], int k) {
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      const float2 t = *reinterpret_cast<const float2*>(x + k + i);
      b[i] = t.x; b[i + 1] = t.y;
    }
  };
  fetch(v, 0);
  int k = 0;
  for (; k + 8 < m; k += 8) {
    float vn[8];
    fetch(vn, k + 8);
#pragma unroll
    for (int i = 0; i < 8; ++i) ss = ss + v[i] * v[i];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = vn[i];
  }
#pragma unroll
  for (int i = 0; i < 8; ++i)
    if (k + i < m) ss = ss + v[i] * v[i];
  return ss;
}

// Dynamic LDS of the one-token append: thresholds, then (STAGE_V) the padded value rotation
// and, with dense rotations, the key groups' matrices (rows padded to m + 1 floats; at most
// d (d + 1) floats in all, the case of a single group).
constexpr int kAppendThrFloats = kMaxBits * 255;
__host__ __device__ inline size_t append_one_lds_bytes(int d, bool stage_v, bool stage_k) {
  return size_t(kAppendThrFloats) * 4 + (stage_v ? size_t(d) * (d + 1) * 4 : 0) +
         (stage_k ? size_t(d) * (d + 1) * 4 : 0);
}

template <typename T, bool STAGE_V, bool WIN, bool GIV>
__device__ __forceinline__ void append_one_wg(const AppendArgs& a, int si, int hk, float* dyn) {
  constexpr int DM = BGTQ_MAX_HEAD_DIM;
  constexpr bool STAGE_K = STAGE_V && !GIV;        // key matrices staged beside the value rotation
  const int d = a.d, bv = a.v_bits;
  float* thr = dyn;                                // [8][255]
  float* rv = dyn + kAppendThrFloats;              // [d][d + 1] (STAGE_V, dense)
  float* rk = rv + d * (d + 1);                    // group g's matrix from rko[g], rows m_g + 1 apart
  __shared__ HeadLayout L;
  __shared__ __align__(16) float ko[DM];           // key, original coordinate order
  __shared__ __align__(16) float xk[2 * DM + 16];  // key, storage order, zero past d_eff
  __shared__ __align__(16) float xv[DM + 16];      // value, zero past d
  __shared__ float nrm[kMaxGroups + 1];            // group norms, value norm last
  __shared__ uint32_t kw[kMaxRecordDwords];        // the slot's key record, assembled with atomic ors
  __shared__ int rko[kMaxGroups + 1];              // float offsets of the staged key matrices
  const int s = a.seq_begin + si, t = threadIdx.x;
  const size_t reg = size_t(s) * a.n_kv_heads + hk;
  const T* kin = static_cast<const T*>(a.keys) + si * a.stride_seq + int64_t(hk) * a.stride_head;
  const T* vin = static_cast<const T*>(a.values) + si * a.stride_seq + int64_t(hk) * a.stride_head;
  // ---- first round of reads: everything that depends neither on the length nor on the layout
  uint4 lw = uint4{0u, 0u, 0u, 0u};
  if (t < 256) lw = reinterpret_cast<const uint4*>(a.layouts + reg)[t];
  const float kval = t < d ? load_f(kin, t) : 0.0f;
  const float vval = t < d ? load_f(vin, t) : 0.0f;
  float tv[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) tv[i] = t + 1024 * i < kAppendThrFloats ? (&c_thr[0][0])[t + 1024 * i] : 0.0f;
  float4 rvq[4];                                  // d <= 128: at most 4096 pieces
  if (STAGE_V && !GIV) {
    const float4* src = reinterpret_cast<const float4*>(a.rot_v);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = t + 1024 * i;
      rvq[i] = q < d * d / 4 ? src[q] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  const int64_t len = a.lengths[s];
  __builtin_amdgcn_sched_barrier(0);      // every read above issued before the first store
  if (t < 256) reinterpret_cast<uint4*>(&L)[t] = lw;
  if (t < DM) { ko[t] = kval; xv[t] = vval; }
  if (t < 16) xv[DM + t] = 0.0f;
#pragma unroll
  for (int i = 0; i < 2; ++i)
    if (t + 1024 * i < kAppendThrFloats) thr[t + 1024 * i] = tv[i];
  if (STAGE_V && !GIV) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = t + 1024 * i;
      if (q < d * d / 4) {
        const int row = (4 * q) / d, col = 4 * q - row * d;
        float* dst = rv + row * (d + 1) + col;
        dst[0] = rvq[i].x; dst[1] = rvq[i].y; dst[2] = rvq[i].z; dst[3] = rvq[i].w;
      }
    }
  }
  if (t < kMaxRecordDwords) kw[t] = 0u;
  __syncthreads();
  if (len + 1 > a.capacity) {                     // the same for every thread
    if (t == 0 && hk == 0 && a.status) atomicOr(a.status, 1);
    return;
  }
  const int64_t tiles = a.capacity / kTile;
  const int64_t tile = len / kTile;
  const int slot = int(len - tile * kTile);
  const uint32_t vmask = (1u << bv) - 1u;
  const int vbit = slot * bv, vw = vbit >> 5, vsh = vbit & 31;
  const bool vsplit = vsh + bv > 32;
  uint32_t* vseg = reinterpret_cast<uint32_t*>(a.v_codes) + (reg * tiles + tile) * d * 2 * bv;
  const int ng = L.n_groups, d_eff = L.d_eff;
  // ---- second round: the slot's old value dwords (by the length), the key matrices (by the layout)
  uint32_t old0 = 0u, old1 = 0u;
  if (t < d) {
    old0 = vseg[t * 2 * bv + vw];
    if (vsplit) old1 = vseg[t * 2 * bv + vw + 1];
  }
  if constexpr (STAGE_K) {
    // group g's m x m matrix (row-major in the bank) to rk + rko[g], rows padded to m + 1
    int pre[kMaxGroups + 1];
    pre[0] = 0;
#pragma unroll
    for (int g = 0; g < kMaxGroups; ++g) pre[g + 1] = pre[g] + (g < ng ? L.g_m[g] * L.g_m[g] : 0);
    if (t <= kMaxGroups) {
      int o = 0;
      for (int g = 0; g < t && g < ng; ++g) o += L.g_m[g] * (L.g_m[g] + 1);
      rko[t] = o;
    }
    constexpr int KQ = 4;                       // float4 pieces per thread (d <= 128: at most 4096)
    float4 kq[KQ];
#pragma unroll
    for (int i = 0; i < KQ; ++i) {
      const int q = t + 1024 * i;
      kq[i] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (4 * q < pre[kMaxGroups]) {
        int g = 0;
#pragma unroll
        for (int gg = 1; gg < kMaxGroups; ++gg) g += 4 * q >= pre[gg] && gg < ng ? 1 : 0;
        const int m = L.g_m[g];
        kq[i] = *reinterpret_cast<const float4*>(a.rot_bank + bank_offset(m) + (4 * q - pre[g]));
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < KQ; ++i) {
      const int q = t + 1024 * i;
      if (4 * q < pre[kMaxGroups]) {
        int g = 0, o = 0;
#pragma unroll
        for (int gg = 1; gg < kMaxGroups; ++gg) g += 4 * q >= pre[gg] && gg < ng ? 1 : 0;
#pragma unroll
        for (int gg = 0; gg < kMaxGroups; ++gg) o += gg < g ? L.g_m[gg] * (L.g_m[gg] + 1) : 0;
        const int m = L.g_m[g], e0 = 4 * q - pre[g];
        // row = e0 / m (e0 < m * m, m <= 128): the exact quotient of e0 + 1/2 is at least 1/(2m)
        // away from an integer, far more than the rounding error of the float division
        int row = int((float(e0) + 0.5f) / float(m)), col = e0 - row * m;
        const float e[4] = {kq[i].x, kq[i].y, kq[i].z, kq[i].w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          rk[o + row * (m + 1) + col] = e[c];
          if (++col == m) { col = 0; ++row; }
        }
      }
    }
  }
  int mmax = 0;
  for (int g = 0; g < ng; ++g) mmax = L.g_m[g] > mmax ? L.g_m[g] : mmax;
  mmax = (mmax + 15) & ~15;
  for (int i = t; i < 2 * DM + 16; i += 1024) xk[i] = i < d_eff ? ko[L.perm[i]] : 0.0f;
  __syncthreads();
  float acc = 0.0f;
  if constexpr (GIV) {
    // structured rotations: norms of the unrotated vectors, then the layers in place
    if (t < ng) nrm[t] = sqrtf(seq_sumsq(xk + L.g_first[t], L.g_m[t]));
    else if (t == ng) nrm[kMaxGroups] = sqrtf(seq_sumsq(xv, d));
    // one pair slot per thread: value slot t, or key slot t - 512 of its width group
    GivensSlot gs;
    gs.n = 0;
    float* gx = nullptr;
    if (t < d / 2) {
      givens_fetch(a.givens, d, t, gs);
      gx = xv;
    } else if (t >= 512 && t < 512 + d_eff / 2) {
      const int q = t - 512, g = L.group[2 * q], first = L.g_first[g];
      givens_fetch(a.givens, L.g_m[g], q - first / 2, gs);
      gx = xk + first;
    }
    const int nl = max(givens_count(a.givens, d), givens_layers(a.givens, L));
    __syncthreads();
#pragma unroll
    for (int l = 0; l < kMaxGivensLayers; ++l) {
      if (l < nl) {
        if (l < gs.n) {
          gs.apply(gx, l);
          if (l + kGivensAhead < kMaxGivensLayers) gs.fetch(l + kGivensAhead);
        }
        __syncthreads();
      }
    }
    if (t < d) acc = xv[t];
    else if (t >= d && t < d + d_eff) acc = xk[t - d];
  } else {
    // norms run beside the rotations
    if (t < d) {                                        // value rotation, row t
      acc = STAGE_V ? dot_rows_lds_any(rv, d + 1, d, t, xv) : dot_rows_t(a.rot_v_t, d, d, t, xv);
    } else if (t >= d && t < d + d_eff) {               // key position p, row p - first of its group
      const int p = t - d, g = L.group[p], m = L.g_m[g], first = L.g_first[g];
      acc = STAGE_K ? dot_rows_lds_any(rk + rko[g], m + 1, m, p - first, xk + first)
                    : dot_rows_t(a.rot_bank_t + bank_offset(m), m, mmax, p - first, xk + first);
    } else if (t >= 768 && t < 768 + ng) {              // group norm
      const int g = t - 768;
      nrm[g] = sqrtf(seq_sumsq(xk + L.g_first[g], L.g_m[g]));
    } else if (t == 768 + kMaxGroups) {                 // value norm
      nrm[kMaxGroups] = sqrtf(seq_sumsq(xv, d));
    }
  }
  __syncthreads();
  // codes: a value code goes straight into the slot's dwords (read before any arithmetic);
  // key codes are ored into the slot's record, assembled in LDS
  if (t < d) {
    const float nv = nrm[kMaxGroups];
    const uint32_t code = nv != 0.0f ? code_of(thr + (bv - 1) * 255, bv, (acc / nv) * sqrtf(float(d))) : 0u;
    vseg[t * 2 * bv + vw] = (old0 & ~(vmask << vsh)) | (code << vsh);
    if (vsplit) vseg[t * 2 * bv + vw + 1] = (old1 & ~(vmask >> (32 - vsh))) | (code >> (32 - vsh));
  } else if (t >= d && t < d + d_eff) {
    const int p = t - d, g = L.group[p], w = L.g_width[g], m = L.g_m[g];
    const float nv = nrm[g];
    const uint32_t code = nv != 0.0f ? code_of(thr + (w - 1) * 255, w, (acc / nv) * sqrtf(float(m))) : 0u;
    const int off = L.offset[p], wd = off >> 5, sh = off & 31;
    atomicOr(&kw[wd], code << sh);
    if (sh + w > 32) atomicOr(&kw[wd + 1], code >> (32 - sh));
  }
  __syncthreads();
  uint32_t* kc = reinterpret_cast<uint32_t*>(a.k_codes) + (reg * tiles + tile) * a.chunks * kTile * 4;
  if (t < 4 * a.chunks) kc[((t >> 2) * kTile + slot) * 4 + (t & 3)] = kw[t];
  uint16_t* kn = a.k_norms + (reg * tiles + tile) * kMaxGroups * kTile;
  if (t >= 256 && t < 256 + ng) kn[(t - 256) * kTile + slot] = f32_to_f16_bits(fminf(nrm[t - 256], 65504.0f));
  if (t == 256 + kMaxGroups)
    a.v_norms[(reg * tiles + tile) * kTile + slot] = f32_to_f16_bits(fminf(nrm[kMaxGroups], 65504.0f));
  // the key's fp16 copy in the recent-key window, last (off the path of the packed stores)
  if (WIN && t >= 1024 - d)
    a.k_window[(reg * a.window + len % a.window) * d + (t - (1024 - d))] = f16_sat_bits(ko[t - (1024 - d)]);
}

template <typename T, bool STAGE_V, bool WIN, bool GIV>
__global__ __launch_bounds__(1024) void k_append_one(AppendArgs a) {
  extern __shared__ __align__(16) float dyn[];
  append_one_wg<T, STAGE_V, WIN, GIV>(a, blockIdx.x / a.n_kv_heads, blockIdx.x % a.n_kv_heads, dyn);
}

// ---- decode step, append role: the one-token append of (sequence s, KV head hk) on one 256-thread
// workgroup of the split kernel, the same arithmetic as k_append_one; the rotations read the
// transposed matrices from global memory.  Once its stores are released, it publishes the new
// length in step_flag[s][hk]; the split that reads the new token's tile waits for that.
constexpr size_t kStepAppendLds =
    size_t(kAppendThrFloats) * 4 + sizeof(HeadLayout) +
    4 * size_t(BGTQ_MAX_HEAD_DIM + 2 * BGTQ_MAX_HEAD_DIM + 16 + BGTQ_MAX_HEAD_DIM + 16 + kMaxGroups + 1 + kMaxRecordDwords);

// Every thread of the workgroup calls it (it holds the barriers); threads from 256 on take
// part in the barriers only.
template <bool WIN, bool GIV>
__device__ void step_append_role(const AppendArgs& a, int32_t* flags, int s, int hk, uint8_t* lds) {
  constexpr int DM = BGTQ_MAX_HEAD_DIM;
  const int t = threadIdx.x, d = a.d, bv = a.v_bits;
  const bool act = t < 256;
  float* thr = reinterpret_cast<float*>(lds);                                   // [8][255]
  HeadLayout* Lp = reinterpret_cast<HeadLayout*>(lds + kAppendThrFloats * 4);
  float* ko = reinterpret_cast<float*>(Lp + 1);        // key, original order
  float* xk = ko + DM;                                 // key, storage order, zero past d_eff
  float* xv = xk + 2 * DM + 16;                        // value, zero past d
  float* nrm = xv + DM + 16;                           // group norms, value norm last
  uint32_t* kw = reinterpret_cast<uint32_t*>(nrm + kMaxGroups + 1);   // the slot's key record
  const size_t reg = size_t(s) * a.n_kv_heads + hk;
  const int si = s - a.seq_begin;
  const size_t esz = a.kv_bf16 ? 2 : 4;
  const char* kin = static_cast<const char*>(a.keys) + (si * a.stride_seq + hk * a.stride_head) * esz;
  const char* vin = static_cast<const char*>(a.values) + (si * a.stride_seq + hk * a.stride_head) * esz;
  auto ld = [&](const char* base, int i) {
    return a.kv_bf16 ? load_f(reinterpret_cast<const uint16_t*>(base), i) : load_f(reinterpret_cast<const float*>(base), i);
  };
  // ---- first round of reads: none depends on the length or on the layout
  const uint4 lw = act ? reinterpret_cast<const uint4*>(a.layouts + reg)[t] : uint4{0u, 0u, 0u, 0u};
  const float kval = t < d ? ld(kin, t) : 0.0f;
  const float vval = t < d ? ld(vin, t) : 0.0f;
  float tv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) tv[i] = act && t + 256 * i < kAppendThrFloats ? (&c_thr[0][0])[t + 256 * i] : 0.0f;
  const int64_t len = a.lengths[s];
  __builtin_amdgcn_sched_barrier(0);
  if (act) {
    reinterpret_cast<uint4*>(Lp)[t] = lw;
    ko[t] = kval;
    xv[t] = vval;
    if (t < 16) xv[DM + t] = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (t + 256 * i < kAppendThrFloats) thr[t + 256 * i] = tv[i];
    if (t < kMaxRecordDwords) kw[t] = 0u;
  }
  __syncthreads();
  if (len + 1 > a.capacity) {                     // nothing appended; the splits do not wait
    if (t == 0 && hk == 0 && a.status) atomicOr(a.status, 1);
    return;
  }
  const HeadLayout& L = *Lp;
  const int64_t tiles = a.capacity / kTile;
  const int64_t tile = len / kTile;
  const int slot = int(len - tile * kTile);
  const uint32_t vmask = (1u << bv) - 1u;
  const int vbit = slot * bv, vw = vbit >> 5, vsh = vbit & 31;
  const bool vsplit = vsh + bv > 32;
  uint32_t* vseg = reinterpret_cast<uint32_t*>(a.v_codes) + (reg * tiles + tile) * d * 2 * bv;
  const int ng = L.n_groups, d_eff = L.d_eff;
  uint32_t old0 = 0u, old1 = 0u;
  if (t < d) {
    old0 = vseg[t * 2 * bv + vw];
    if (vsplit) old1 = vseg[t * 2 * bv + vw + 1];
  }
  int mmax = 0;
  for (int g = 0; g < ng; ++g) mmax = L.g_m[g] > mmax ? L.g_m[g] : mmax;
  mmax = (mmax + 15) & ~15;
  if (act)
    for (int i = t; i < 2 * DM + 16; i += 256) xk[i] = i < d_eff ? ko[L.perm[i]] : 0.0f;
  __syncthreads();
  // rotations: value row r < d, key position r - d; rows t and t + 256
  float acc[2] = {0.0f, 0.0f};
  if constexpr (GIV) {
    if (t < ng) nrm[t] = sqrtf(seq_sumsq(xk + L.g_first[t], L.g_m[t]));
    else if (t == ng) nrm[kMaxGroups] = sqrtf(seq_sumsq(xv, d));
    // one pair slot per thread: value slot t, or key slot t - 128 of its width group
    GivensSlot gs;
    gs.n = 0;
    float* gx = nullptr;
    if (t < d / 2) {
      givens_fetch(a.givens, d, t, gs);
      gx = xv;
    } else if (t >= 128 && t < 128 + d_eff / 2) {
      const int q = t - 128, g = L.group[2 * q], first = L.g_first[g];
      givens_fetch(a.givens, L.g_m[g], q - first / 2, gs);
      gx = xk + first;
    }
    const int nl = max(givens_count(a.givens, d), givens_layers(a.givens, L));
    __syncthreads();
#pragma unroll
    for (int l = 0; l < kMaxGivensLayers; ++l) {
      if (l < nl) {
        if (l < gs.n) {
          gs.apply(gx, l);
          if (l + kGivensAhead < kMaxGivensLayers) gs.fetch(l + kGivensAhead);
        }
        __syncthreads();
      }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int r = t + 256 * j;
      if (r < d) acc[j] = xv[r];
      else if (r < d + d_eff) acc[j] = xk[r - d];
    }
  } else {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int r = t + 256 * j;
      if (r < d) {
        acc[j] = dot_rows_t(a.rot_v_t, d, d, r, xv);
      } else if (r < d + d_eff) {
        const int p = r - d, g = L.group[p], m = L.g_m[g], first = L.g_first[g];
        acc[j] = dot_rows_t(a.rot_bank_t + bank_offset(m), m, mmax, p - first, xk + first);
      }
    }
    if (t < ng) nrm[t] = sqrtf(seq_sumsq(xk + L.g_first[t], L.g_m[t]));
    else if (t == ng) nrm[kMaxGroups] = sqrtf(seq_sumsq(xv, d));
  }
  __syncthreads();
  // codes: a value code goes straight into the slot's dwords; key codes are ored into the record
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = t + 256 * j;
    if (!act) {
    } else if (r < d) {
      const float nv = nrm[kMaxGroups];
      const uint32_t code = nv != 0.0f ? code_of(thr + (bv - 1) * 255, bv, (acc[j] / nv) * sqrtf(float(d))) : 0u;
      vseg[r * 2 * bv + vw] = (old0 & ~(vmask << vsh)) | (code << vsh);
      if (vsplit) vseg[r * 2 * bv + vw + 1] = (old1 & ~(vmask >> (32 - vsh))) | (code >> (32 - vsh));
    } else if (r < d + d_eff) {
      const int p = r - d, g = L.group[p], w = L.g_width[g], m = L.g_m[g];
      const float nv = nrm[g];
      const uint32_t code = nv != 0.0f ? code_of(thr + (w - 1) * 255, w, (acc[j] / nv) * sqrtf(float(m))) : 0u;
      const int off = L.offset[p], wd = off >> 5, sh = off & 31;
      atomicOr(&kw[wd], code << sh);
      if (sh + w > 32) atomicOr(&kw[wd + 1], code >> (32 - sh));
    }
  }
  __syncthreads();
  uint32_t* kc = reinterpret_cast<uint32_t*>(a.k_codes) + (reg * tiles + tile) * a.chunks * kTile * 4;
  if (t < 4 * a.chunks) kc[((t >> 2) * kTile + slot) * 4 + (t & 3)] = kw[t];
  uint16_t* kn = a.k_norms + (reg * tiles + tile) * kMaxGroups * kTile;
  if (t < ng) kn[t * kTile + slot] = f32_to_f16_bits(fminf(nrm[t], 65504.0f));
  if (t == 255) a.v_norms[(reg * tiles + tile) * kTile + slot] = f32_to_f16_bits(fminf(nrm[kMaxGroups], 65504.0f));
  if (WIN && t < d) a.k_window[(reg * a.window + len % a.window) * d + t] = f16_sat_bits(ko[t]);
  // ---- publish: every store released at device scope, then the new length
  __threadfence();
  __syncthreads();
  if (t == 0) __hip_atomic_store(flags + reg, int32_t(len + 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}


// fp16 keys of the appended tokens that end up among the newest `window` (the last
// min(n_new, window) of them), at slot t % window; runs before the length advance.
template <typename T>
__global__ __launch_bounds__(256) void k_window_store(AppendArgs a) {
  const int si = blockIdx.z, s = a.seq_begin + si, hk = blockIdx.y;
  const int64_t len = a.lengths[s];
  if (len + a.n_new > a.capacity) return;          // the append itself is skipped
  const int64_t m = a.n_new < a.window ? a.n_new : a.window;
  const int64_t idx = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= m * a.d) return;
  const int64_t i = a.n_new - m + idx / a.d;       // token of the append
  const int c = int(idx % a.d);
  const T* kin = static_cast<const T*>(a.keys) + si * a.stride_seq + int64_t(hk) * a.stride_head;
  const size_t reg = size_t(s) * a.n_kv_heads + hk;
  a.k_window[(reg * a.window + (len + i) % a.window) * a.d + c] = f16_sat_bits(load_f(kin, i * a.stride_token + c));
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

// Query prologue of the vector-ALU kernel: q' = RoPE(q, pos) for the G query heads of one
// (sequence, KV head) with fp64 angles, then q'' for storage positions p of the head's layout,
//   q''[h][p] = (softmax_scale * log2(e) / sqrt(m)) * sum_k R_m[p - first][k] q'[h][perm[first + k]],
// m and first those of p's width group, so that logits come out in base-2 units.  Workgroup
// z of the (sequence, KV head) writes fp32 q'' [position][kQPad] of positions z, z + kPrepZ, ..
// (the matrix-core kernel computes the same quantity in its own prologue).
constexpr int kPrepZ = 8;
template <typename T>
__global__ __launch_bounds__(256) void k_decode_prep(DecodeArgs a) {
  __shared__ HeadLayout L;
  __shared__ float qs[BGTQ_MAX_GROUP * BGTQ_MAX_HEAD_DIM];          // q' by coordinate
  __shared__ float qp[BGTQ_MAX_GROUP * (BGTQ_MAX_HEAD_DIM + 1)];    // q' by storage position
  const int hk = blockIdx.x, s = blockIdx.y, z = blockIdx.z, tid = threadIdx.x;
  const int G = a.group, d = a.d, n = d / 2, QS = d + 1;
  {
    const uint4* src = reinterpret_cast<const uint4*>(a.layouts + int64_t(s) * a.n_kv + hk);
    uint4* dst = reinterpret_cast<uint4*>(&L);
    for (int i = tid; i < int(sizeof(HeadLayout) / 16); i += 256) dst[i] = src[i];
  }
  const int64_t pos = a.q_pos ? a.q_pos[s] : int64_t(a.lengths[s]) - 1;
  const T* q = static_cast<const T*>(a.q) + (int64_t(s) * a.n_q + int64_t(hk) * G) * d;
  for (int idx = tid; idx < G * n; idx += 256) {
    const int h = idx / n, j = idx - h * n;
    const int ca = a.pairing ? 2 * j : j, cb = a.pairing ? 2 * j + 1 : j + n;
    const double x0 = load_f(q + int64_t(h) * d, ca), x1 = load_f(q + int64_t(h) * d, cb);
    double sv = 0.0, cv = 1.0;
    if (a.rope_theta > 0.0) sincos(fmod(double(pos) * a.inv_freq[j], kTwoPi), &sv, &cv);
    qs[h * d + ca] = float(x0 * cv - x1 * sv);
    qs[h * d + cb] = float(x0 * sv + x1 * cv);
  }
  __syncthreads();
  const int d_eff = L.d_eff;
  for (int idx = tid; idx < G * d_eff; idx += 256) {
    const int h = idx / d_eff, p = idx - h * d_eff;
    qp[h * QS + p] = qs[h * d + L.perm[p]];
  }
  __syncthreads();
  if (a.givens) {   // structured rotations: every group of every head in place, layer by layer
    const int nl = givens_layers(a.givens, L);
    for (int l = 0; l < nl; ++l) {
      for (int idx = tid; idx < G * (d_eff / 2); idx += 256) {
        const int h = idx / (d_eff / 2), q = idx - h * (d_eff / 2);
        uint4 rec;
        int first;
        if (givens_slot(a.givens, L, q, l, rec, first)) givens_pair(qp + h * QS + first, rec);
      }
      __syncthreads();
    }
  }
  const float kscale = a.scale * kLog2e;
  // q'' of position p and head h: the group's rotation row times q' (fp32 fused multiply-adds),
  // or the rotated q' itself for structured rotations
  auto qpp = [&](int p, int h) {
    const int g = L.group[p], m = L.g_m[g], first = L.g_first[g];
    if (a.givens) return qp[h * QS + p] * (kscale / sqrtf(float(m)));
    const float2* R2 = reinterpret_cast<const float2*>(a.rot_bank + bank_offset(m) + size_t(p - first) * m);
    const float* x = qp + h * QS + first;
    float acc = 0.0f;
#pragma unroll 16
    for (int k = 0; k < m; k += 2) {
      const float2 r = R2[k >> 1];
      acc = fmaf(r.x, x[k], acc);
      acc = fmaf(r.y, x[k + 1], acc);
    }
    return acc * (kscale / sqrtf(float(m)));
  };
  {   // fp32 [position][kQPad], zero past d_eff and G
    float* dst = a.qrot + (int64_t(s) * a.n_kv + hk) * d * kQPad;
    for (int idx = tid; idx < ((d - z + kPrepZ - 1) / kPrepZ) * kQPad; idx += 256) {
      const int p = z + kPrepZ * (idx / kQPad), h = idx % kQPad;
      dst[p * kQPad + h] = (p < d_eff && h < G) ? qpp(p, h) : 0.0f;
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
    cbk[i] = c_cen[w - 1][i + 2 - (1 << w)];   // fp32 levels
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
    const int64_t row = (int64_t(s) * a.n_q + hk * a.group + h) * a.n_split + split;
    float* dst = a.partial + row * D;
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
      if (c < D) dst[c] = v;
      else reinterpret_cast<float*>(a.part_ml + row)[c - D] = v;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- matrix-core split-K pass
// Same partial results as k_decode_split, with both contractions on MFMA
// (v_mfma_f32_16x16x32_f16, fp32 accumulation).  The four wavefronts of a workgroup work on
// one 64-token tile at a time:
//   keys    wave w owns tokens 16 w .. 16 w + 15 (the 16 rows of its A operand); its lane
//           (n, j) decodes 8 codes of token 16 w + n for k-step s from segment 4 s + j of the
//           token's K record; B is the rotated query (columns 0-7: the G heads restricted
//           to the k-step's first width group, columns 8-15: its second group) as an fp16
//           high part (registers) and an fp16 remainder (LDS), two MFMAs; each column
//           half's partial logit is scaled by its group's fp32 norm, and column c + column
//           c + 8 is head c.
//   softmax the tile maximum per head is shared through LDS; p * n_v goes to LDS as the fp16
//           B operand of P V (lane group j of sub-tile st holds tokens 32 st + 8 j .. + 7).
//   values  wave w owns rotated coordinates D/4 w .. D/4 (w + 1) - 1; A rows are coordinates,
//           each lane decodes 8 consecutive tokens of one coordinate.
// Codes become fp16 levels through pair tables (two codes of width w <= 4 index one packed
// half2) or, for k-steps with a wider segment, single-level tables of every width.  Every wave
// stages only the bytes it reads (its tokens' K records and norms, its coordinates' value
// segments); the next tile's loads go to registers while the current tile is computed.
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kQRegSteps = 8;        // k-steps whose query operands stay in registers

__device__ __forceinline__ int pair_base(int w) { return ((1 << (2 * w)) - 4) / 3; }
__device__ __forceinline__ int single_base(int w) { return (1 << w) - 2; }

// Per-wave staging of one tile (bytes): K records of the wave's 16 tokens [token][chunk][16 B],
// group norms and value norms [g][16] fp16 (value norms at g = n_groups), value segments of
// the wave's D/4 coordinates [coord][8 b_v B].
struct TcStage {
  int n_off, v_off, bytes;
};
__host__ __device__ inline TcStage tc_stage(int D, int chunks, int bv) {
  TcStage g;
  g.n_off = 256 * chunks;
  g.v_off = g.n_off + 16 * (2 * kMaxGroups + 2);
  g.bytes = (g.v_off + 2 * D * bv + 255) & ~255;
  return g;
}
// Workgroup LDS (bytes): tables, k-step descriptors, P operands, softmax exchange, ring.
constexpr int kTcTab = (8 * kPairWords + 4 * kSingleHalves + 15) & ~15;   // 12960: hi/lo pairs, hi | lo singles
constexpr int kTcDesc = kTcTab;                                       // uint4 [kMaxKSteps][4]
constexpr int kTcNorm = kTcDesc + 16 * 4 * kMaxKSteps;                // uint32 [kMaxKSteps]
constexpr int kTcP = (kTcNorm + 4 * kMaxKSteps + 15) & ~15;           // [2][64][16 B]
constexpr int kTcMx = kTcP + 2048;                                    // float [8][16] maxima, [4][8] sums
constexpr int kTcRing = (kTcMx + 4 * (128 + 32) + 255) & ~255;
// Largest k-step count of a layout: 5, 7 and 11 for head dims 64, 128 and 256 (exhaustive
// over the segment counts that width groups of those dims can have), so only head dim 256
// has k-steps past the register-resident ones.
__host__ __device__ constexpr int tc_ksteps(int D) { return D / 32 + 3; }
// The query prologue's copy of the layout descriptor, q' [coordinate][8 heads] and the high
// parts of the register-resident k-steps' B operands [k-step][64 lanes][16 B] alias the ring
// (first written inside the tile loop, after those operands are in registers).  After the
// ring: the low parts of the register-resident k-steps, then both parts of later k-steps.
__host__ __device__ constexpr int tc_qhi_off(int D) { return BGTQ_LAYOUT_BYTES + 32 * D; }   // from the ring
__host__ __device__ inline int tc_qlo_off(int D, int chunks, int bv) {
  const int ring = 4 * tc_stage(D, chunks, bv).bytes, pro = tc_qhi_off(D) + 1024 * kQRegSteps;
  return (kTcRing + (ring > pro ? ring : pro) + 255) & ~255;
}
__host__ __device__ inline int tc_lds_bytes(int D, int chunks, int bv) {
  const int later = tc_ksteps(D) > kQRegSteps ? tc_ksteps(D) - kQRegSteps : 0;
  return tc_qlo_off(D, chunks, bv) + 1024 * kQRegSteps + 2048 * later;
}

__device__ __forceinline__ uint32_t lds_u32(const uint8_t* base, uint32_t off) {
  return *reinterpret_cast<const uint32_t*>(base + off);
}

// Eight consecutive codes of width w starting at bit sh of the window d2:d1:d0, as fp16 levels
// hi (h) and lo (l), hi + lo = the fp32 level to about 2^-22 (low half = first code).  tb = byte
// offset of the width's table in LDS: the hi/lo pair table (w <= 5) or the hi | lo single table.
__device__ __forceinline__ void decode8(uint32_t d0, uint32_t d1, uint32_t d2, int sh, int w, const uint8_t* lds,
                                        uint32_t tb, u32x4& h, u32x4& l) {
  if (w <= 4) {      // 8 codes fit one 32-bit window
    const uint32_t x = __builtin_amdgcn_alignbit(d1, d0, sh);
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
      const uint2 v = *reinterpret_cast<const uint2*>(lds + tb + 8 * __builtin_amdgcn_ubfe(x, 2 * e2 * w, 2 * w));
      h[e2] = v.x;
      l[e2] = v.y;
    }
  } else {
    const uint32_t lo = __builtin_amdgcn_alignbit(d1, d0, sh);
    const uint32_t hi = __builtin_amdgcn_alignbit(d2, d1, sh);
    const uint64_t x = (uint64_t(hi) << 32) | lo;
    if (w == 5) {
      const uint32_t mask = 0x3ffu;
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const uint2 v = *reinterpret_cast<const uint2*>(lds + tb + 8 * (uint32_t(x >> (10 * e2)) & mask));
        h[e2] = v.x;
        l[e2] = v.y;
      }
    } else {
      const uint32_t mask = (1u << w) - 1u;
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const uint32_t c0 = uint32_t(x >> (2 * e2 * w)) & mask;
        const uint32_t c1 = uint32_t(x >> ((2 * e2 + 1) * w)) & mask;
        const uint32_t v0 = lds_u32(lds, tb + 4 * c0), v1 = lds_u32(lds, tb + 4 * c1);
        h[e2] = __builtin_amdgcn_perm(v1, v0, 0x05040100u);
        l[e2] = __builtin_amdgcn_perm(v1, v0, 0x07060302u);
      }
    }
  }
}

// Eight consecutive codes of any width w (1..8) starting at bit sh of the window d2:d1:d0, as
// fp16 levels hi and lo from the width's hi | lo single table at byte offset tb (low half =
// first code).  One instruction sequence for every width, so lanes whose segments differ in
// width run it together instead of one width class after another.
__device__ __forceinline__ void decode8_any(uint32_t d0, uint32_t d1, uint32_t d2, int sh, int w, const uint8_t* lds,
                                            uint32_t tb, u32x4& h, u32x4& l) {
  const uint64_t x = (uint64_t(__builtin_amdgcn_alignbit(d2, d1, sh)) << 32) | __builtin_amdgcn_alignbit(d1, d0, sh);
  const uint32_t mask = (1u << w) - 1u;
#pragma unroll
  for (int e2 = 0; e2 < 4; ++e2) {
    const uint32_t c0 = uint32_t(x >> (2 * e2 * w)) & mask;
    const uint32_t c1 = uint32_t(x >> ((2 * e2 + 1) * w)) & mask;
    const uint32_t v0 = lds_u32(lds, tb + 4 * c0), v1 = lds_u32(lds, tb + 4 * c1);
    h[e2] = __builtin_amdgcn_perm(v1, v0, 0x05040100u);
    l[e2] = __builtin_amdgcn_perm(v1, v0, 0x07060302u);
  }
}

// Workgroup barrier that orders LDS only: waits for this wave's LDS operations, not for its
// outstanding global loads, so staging loads for later tiles stay in flight across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// ---- rotated query, formed in the matrix-core kernel's prologue.  q' = RoPE(q, pos) with the angle formed and reduced modulo 2 pi in fp64;
// q''[h][p] = (softmax_scale * log2(e) / sqrt(m)) * sum_k R_m[p - first][k] q'[h][perm[first + k]]
// (m and first of storage position p's width group), split into an fp16 high part and an fp16
// remainder and scattered into the B operand layout: lane 16 j + c of k-step s holds k indices
// 32 s + 8 j + e, column c < 8 is head c for the k-step's first width group, c + 8 head c for
// its second; every other entry (other column half, heads >= G, unused k indices) is 0.  The
// helpers run on 256 threads (tid < 256).
template <int D>
struct QShape {
  static constexpr int NP = D / 2;
  static constexpr int QI = 8 * NP / 256 > 0 ? 8 * NP / 256 : 1;   // (head, pair) items per thread
  static constexpr int RR = D / 4 < 16 ? D / 4 : 16;                // rotation-row float2 per batch
};

// q of the thread's items (head h, pair jx): idx = tid + 256 it, jx = idx % NP, h = idx / NP;
// zero for heads >= G
template <int D, typename QT>
__device__ __forceinline__ void q_load(const DecodeArgs& a, int s, int hk, int tid, float (&x0)[QShape<D>::QI],
                                       float (&x1)[QShape<D>::QI]) {
  constexpr int NP = QShape<D>::NP;
  static_assert(256 % NP == 0 || NP % 256 == 0, "pair index of a thread's items");
  const QT* qg = static_cast<const QT*>(a.q) + (int64_t(s) * a.n_q + int64_t(hk) * a.group) * D;
#pragma unroll
  for (int it = 0; it < QShape<D>::QI; ++it) {
    const int idx = tid + 256 * it, jx = idx % NP, h = idx / NP;
    x0[it] = 0.0f;
    x1[it] = 0.0f;
    if (h < a.group) {
      x0[it] = load_f(qg + h * D, a.pairing ? 2 * jx : jx);
      x1[it] = load_f(qg + h * D, a.pairing ? 2 * jx + 1 : jx + NP);
    }
  }
}

// q' of the thread's items into qc [coordinate][8 heads]; fr = inv_freq[tid % NP]
template <int D>
__device__ __forceinline__ void q_rope(const DecodeArgs& a, int64_t pos, double fr, int tid,
                                       const float (&x0)[QShape<D>::QI], const float (&x1)[QShape<D>::QI], float* qc) {
  constexpr int NP = QShape<D>::NP;
  float cv = 1.0f, sv = 0.0f;
  if (a.rope_theta > 0.0) {
    const double ang = double(pos) * fr;
    sincosf(float(ang - kTwoPi * floor(ang * (1.0 / kTwoPi))), &sv, &cv);
  }
#pragma unroll
  for (int it = 0; it < QShape<D>::QI; ++it) {
    const int idx = tid + 256 * it, jx = idx % NP, h = idx / NP;
    if (h < 8) {
      const double a0 = x0[it], a1 = x1[it];   // zero for heads >= G
      qc[8 * (a.pairing ? 2 * jx : jx) + h] = float(a0 * cv - a1 * sv);
      qc[8 * (a.pairing ? 2 * jx + 1 : jx + NP) + h] = float(a0 * sv + a1 * cv);
    }
  }
}

// The matrix-core kernel takes the layout's k-steps in a different order: the narrow ones
// (every segment at most 4 bits wide) first, in layout order, then the wide ones.  The mask
// marks the layout's wide k-steps (a ballot: every lane of the wave takes part).
__device__ __forceinline__ uint32_t wide_ksteps(const HeadLayout* Ls, int nks, int lane) {
  bool wd = false;
  if (lane < nks) {
    const uint4 sg = reinterpret_cast<const uint4*>(Ls->seg)[lane];   // the k-step's four segments, one read
    const uint32_t w = max(max((sg.x >> 16) & 15u, (sg.y >> 16) & 15u), max((sg.z >> 16) & 15u, (sg.w >> 16) & 15u));
    wd = w > 4u;
  }
  return uint32_t(__ballot(wd));
}
// place of layout k-step ks in the kernel's order (nn narrow k-steps)
__device__ __forceinline__ int kperm_of(uint32_t wmask, int nn, int ks) {
  const int below = __popc(wmask & ((1u << ks) - 1u));
  return ((wmask >> ks) & 1u) ? nn + below : ks - below;
}

// B operand storage: high parts of k-steps < 8 [ks][lane], their remainders [ks][lane], both
// parts of later k-steps [ks - 8][hi, lo][lane]
__device__ __forceinline__ void qops_zero(uint4* qhi, uint4* qlo, uint4* qlate, int nks, int tid) {
  for (int i = tid; i < 64 * nks; i += 256) {
    const uint4 z = uint4{0u, 0u, 0u, 0u};
    if (i < 64 * kQRegSteps) {
      qhi[i] = z;
      qlo[i] = z;
    } else {
      qlate[2 * (i - 64 * kQRegSteps) - (i & 63)] = z;            // [ks - 8][0][lane]
      qlate[2 * (i - 64 * kQRegSteps) - (i & 63) + 64] = z;       // [ks - 8][1][lane]
    }
  }
}

// q'' of storage position p = p0 + tid / 2 (every 128 positions): the thread pair splits the
// rotation row in two halves and covers all 8 heads, then each thread scatters 4 heads.
// qc = q' [coordinate][8 heads] and the layout copy Ls are in LDS.
// q'' of storage position p for heads 4 kh .. 4 kh + 3 (v) into the B operand slots of its
// k-step, fp16 high part and remainder; heads >= G stay zero.  IL: the streamed pass's layout,
// qhi = k indices e = 0..3 of a lane's 8, qlo = e = 4..7, each as 4 high parts then 4 remainders.
template <bool IL = false>
__device__ __forceinline__ void qops_put(const HeadLayout* Ls, uint32_t wmask, int nn, int p, int kh, int G,
                                         const float (&v)[4], uint4* qhi, uint4* qlo, uint4* qlate) {
  const int kx = Ls->kpos[p], ks0 = kx >> 5, jj = (kx >> 3) & 3, e = kx & 7, ks = kperm_of(wmask, nn, ks0);
  const int lb = 16 * jj + 8 * int((Ls->seg[4 * ks0 + jj] >> 28) & 1u);
  if constexpr (IL) {
    uint16_t* q16 = reinterpret_cast<uint16_t*>((e < 4 ? qhi : qlo) + 64 * ks);
#pragma unroll
    for (int hh = 0; hh < 4; ++hh) {
      const int h = 4 * kh + hh;
      if (h < G) {
        const uint16_t hi = f32_to_f16_bits(v[hh]);
        q16[(lb + h) * 8 + (e & 3)] = hi;
        q16[(lb + h) * 8 + 4 + (e & 3)] = f32_to_f16_bits(v[hh] - f16_bits_to_f32(hi));
      }
    }
    return;
  }
  uint16_t* h16 = reinterpret_cast<uint16_t*>(ks < kQRegSteps ? qhi + 64 * ks : qlate + 128 * (ks - kQRegSteps));
  uint16_t* l16 = reinterpret_cast<uint16_t*>(ks < kQRegSteps ? qlo + 64 * ks : qlate + 128 * (ks - kQRegSteps) + 64);
#pragma unroll
  for (int hh = 0; hh < 4; ++hh) {
    const int h = 4 * kh + hh;
    if (h < G) {
      const uint16_t hi = f32_to_f16_bits(v[hh]);
      h16[(lb + h) * 8 + e] = hi;
      l16[(lb + h) * 8 + e] = f32_to_f16_bits(v[hh] - f16_bits_to_f32(hi));
    }
  }
}

template <int D, bool IL = false>
__device__ __forceinline__ void qops_scatter(const DecodeArgs& a, const HeadLayout* Ls, const float* qc, uint32_t wmask,
                                             int nn, int tid, uint4* qhi, uint4* qlo, uint4* qlate) {
  constexpr int RR = QShape<D>::RR;
  const int d_eff = Ls->d_eff, kh = tid & 1, G = a.group;
  const float kscale = a.scale * kLog2e;
  float2 rr[RR];
  for (int p0 = 0; p0 < d_eff; p0 += 128) {
    const int p = p0 + (tid >> 1);
    int m = 2, first = 0;
    const float2* R2 = nullptr;
    if (p < d_eff) {
      const int g = Ls->group[p];
      m = Ls->g_m[g];
      first = Ls->g_first[g];
      R2 = reinterpret_cast<const float2*>(a.rot_bank + bank_offset(m) + size_t(p - first) * m) + kh * (m / 4);
    }
    const int nh = p < d_eff ? (kh == 0 ? m / 4 : m / 2 - m / 4) : 0;   // float2 of this half
    const uint8_t* pm = Ls->perm + first + 2 * kh * (m / 4);           // its coordinates
    float acc[8];
#pragma unroll
    for (int h = 0; h < 8; ++h) acc[h] = 0.0f;
    for (int b0 = 0; b0 < nh; b0 += RR) {         // one batch unless m > 4 RR
#pragma unroll
      for (int i = 0; i < RR; ++i)
        if (b0 + i < nh) rr[i] = R2[b0 + i];
#pragma unroll
      for (int i = 0; i < RR; ++i) {
        if (b0 + i < nh) {
          const float4* xa = reinterpret_cast<const float4*>(qc + 8 * pm[2 * (b0 + i)]);
          const float4* xb = reinterpret_cast<const float4*>(qc + 8 * pm[2 * (b0 + i) + 1]);
          const float4 a0 = xa[0], a1 = xa[1], c0 = xb[0], c1 = xb[1];
          const float r0 = rr[i].x, r1 = rr[i].y;
          acc[0] = fmaf(r0, a0.x, acc[0]); acc[1] = fmaf(r0, a0.y, acc[1]);
          acc[2] = fmaf(r0, a0.z, acc[2]); acc[3] = fmaf(r0, a0.w, acc[3]);
          acc[4] = fmaf(r0, a1.x, acc[4]); acc[5] = fmaf(r0, a1.y, acc[5]);
          acc[6] = fmaf(r0, a1.z, acc[6]); acc[7] = fmaf(r0, a1.w, acc[7]);
          acc[0] = fmaf(r1, c0.x, acc[0]); acc[1] = fmaf(r1, c0.y, acc[1]);
          acc[2] = fmaf(r1, c0.z, acc[2]); acc[3] = fmaf(r1, c0.w, acc[3]);
          acc[4] = fmaf(r1, c1.x, acc[4]); acc[5] = fmaf(r1, c1.y, acc[5]);
          acc[6] = fmaf(r1, c1.z, acc[6]); acc[7] = fmaf(r1, c1.w, acc[7]);
        }
      }
    }
    // the pair's two halves, lower coordinates first; this thread keeps heads 4 kh .. 4 kh + 3
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float mine = acc[4 * kh + e], give = acc[4 * (1 - kh) + e];
      const float other = __shfl_xor(give, 1);
      v[e] = (kh == 0 ? mine + other : other + mine) * (kscale / sqrtf(float(m)));
    }
    if (p < d_eff) qops_put<IL>(Ls, wmask, nn, p, kh, G, v, qhi, qlo, qlate);
  }
}

// Structured rotations of q' (qc [coordinate][8 heads]) into every width group's frame, in
// place: the pair slots of a group act on original coordinates perm[first + a] and
// perm[first + b]; thread tid < d_eff takes pair slot tid / 2 and four heads (nt >= d_eff
// threads).  Every thread of the workgroup calls it (it holds the barriers).
__device__ __forceinline__ void qops_givens_rotate(const DecodeArgs& a, const HeadLayout* Ls, float* qc, int tid,
                                                   int nt) {
  const int d_eff = Ls->d_eff, q = tid >> 1;        // thread: pair slot q, heads 4 (tid & 1) ..
  GivensSlot gs;
  gs.n = 0;
  int first = 0;
  if (tid < d_eff && tid < nt) {
    const int g = Ls->group[2 * q];
    first = Ls->g_first[g];
    givens_fetch(a.givens, Ls->g_m[g], q - first / 2, gs);
  }
  const int nl = givens_layers(a.givens, *Ls);
#pragma unroll
  for (int l = 0; l < kMaxGivensLayers; ++l) {
    if (l < nl) {
      if (l < gs.n) {
        const int k = l % kGivensAhead;
        const int ca = Ls->perm[first + int(gs.ab[k] & 0xffffu)], cb = Ls->perm[first + int(gs.ab[k] >> 16)];
        const float c = gs.c[k], sn = gs.s[k];
        float4* pa = reinterpret_cast<float4*>(qc + 8 * ca + 4 * (tid & 1));
        float4* pb = reinterpret_cast<float4*>(qc + 8 * cb + 4 * (tid & 1));
        const float4 xa = *pa, xb = *pb;
        *pa = float4{fmaf(c, xa.x, -sn * xb.x), fmaf(c, xa.y, -sn * xb.y), fmaf(c, xa.z, -sn * xb.z),
                     fmaf(c, xa.w, -sn * xb.w)};
        *pb = float4{fmaf(sn, xa.x, c * xb.x), fmaf(sn, xa.y, c * xb.y), fmaf(sn, xa.z, c * xb.z),
                     fmaf(sn, xa.w, c * xb.w)};
        if (l + kGivensAhead < kMaxGivensLayers) gs.fetch(l + kGivensAhead);
      }
      __syncthreads();
    }
  }
}

// B operands from q' already rotated into the group frames (qops_givens_rotate):
// q''_p = q'[perm[p]] * softmax_scale * log2(e) / sqrt(m); 256 threads, as qops_scatter.
template <bool IL = false>
__device__ __forceinline__ void qops_scatter_rotated(const DecodeArgs& a, const HeadLayout* Ls, const float* qc,
                                                     uint32_t wmask, int nn, int tid, uint4* qhi, uint4* qlo,
                                                     uint4* qlate) {
  const int d_eff = Ls->d_eff, kh = tid & 1, G = a.group;
  const float kscale = a.scale * kLog2e;
  for (int p0 = 0; p0 < d_eff; p0 += 128) {
    const int p = p0 + (tid >> 1);
    if (p < d_eff) {
      const float f = kscale / sqrtf(float(Ls->g_m[Ls->group[p]]));
      const float4 x = *reinterpret_cast<const float4*>(qc + 8 * Ls->perm[p] + 4 * kh);
      const float v[4] = {x.x * f, x.y * f, x.z * f, x.w * f};
      qops_put<IL>(Ls, wmask, nn, p, kh, G, v, qhi, qlo, qlate);
    }
  }
}

template <int D, bool NARROW, typename QT, bool STEP, bool WIN>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void k_decode_mfma(DecodeArgs a, AppendArgs aa) {
  constexpr int CPW = D / 4;                          // value coordinates per wave
  constexpr int MTV = CPW / 16;                       // value M-tiles per wave
  constexpr int MAXNK = NARROW ? 1 : (D + 63) / 64;                  // K staging loads per lane
  constexpr int MAXNV = NARROW ? (D / 2 + 63) / 64 : (D + 63) / 64;  // value staging loads per lane
  extern __shared__ __align__(16) uint8_t lds[];
  if constexpr (STEP) {
    // decode step: workgroup 0 of every (sequence, KV head) appends the new token
    if (blockIdx.x == 0) {
      if (aa.givens) step_append_role<WIN, true>(aa, a.step_flag, blockIdx.z, blockIdx.y, lds);
      else step_append_role<WIN, false>(aa, a.step_flag, blockIdx.z, blockIdx.y, lds);
      return;
    }
  }
  const int split = int(blockIdx.x) - (STEP ? 1 : 0), hk = blockIdx.y, s = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, j = lane >> 4;
  // in a decode step the append role adds the new token beside this pass and the merge kernel
  // advances lengths[], so it still holds the old length here
  const int len0 = a.lengths[s];
  const int len = a.step && len0 + 1 <= a.capacity ? len0 + 1 : len0;
  // Tokens [0, pend) are attended from the packed keys by the last n_split - n_wsplit
  // splits; with a window (WIN), the window's tokens [pend, len) from their fp16 keys by the
  // first n_wsplit splits (workgroup-uniform role; dispatched first, as their prologue is the
  // longer one).  Packed split i of n takes tiles i, i + n, i + 2n, ... of the role's T tiles,
  // so its first tile is known before the length is; window split i takes the range
  // [i T / n, (i + 1) T / n).  Either way the counts differ by at most one.
  const int pend = !WIN ? len : (len > a.window ? len - a.window : 0);
  const int nw = WIN ? a.n_wsplit : 0, n_ps = a.n_split - nw;
  const bool win = WIN && split < nw;
  int tbase, tstride, count, vlo, vhi;               // tiles tbase + it * tstride, the role's tokens
  if (!win) {
    const int tiles = (pend + kTile - 1) / kTile;
    tbase = split - nw;
    tstride = n_ps;
    count = tiles > tbase ? (tiles - tbase + n_ps - 1) / n_ps : 0;
    vlo = 0;
    vhi = pend;
  } else {
    const int first = pend / kTile, tiles = pend < len ? (len + kTile - 1) / kTile - first : 0;
    const int nwd = nw > 0 ? nw : 1;               // nw > 0 whenever this role runs
    tbase = first + int(int64_t(split) * tiles / nwd);
    tstride = 1;
    count = first + int(int64_t(split + 1) * tiles / nwd) - tbase;
    vlo = pend;
    vhi = len;
  }
  // decode step: the split whose tiles include the new token's waits for the append role before
  // it requests that tile (iteration it_new), with a bounded wait
  int it_new = -1;
  if constexpr (STEP) {
    if (len == len0 + 1) {
      const int dt = len0 / kTile - tbase;
      if (dt >= 0 && dt % tstride == 0 && dt / tstride < count) it_new = dt / tstride;
    }
  }
  auto wait_append = [&]() {
    if (tid == 0) {
      const int32_t* f = a.step_flag + (size_t(s) * a.n_kv + hk);
      int i = 0;
      for (; i < a.step_spin; ++i) {
        if (__hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == len0 + 1) break;
        __builtin_amdgcn_s_sleep(2);
      }
      if (i == a.step_spin && aa.status) atomicOr(aa.status, 2);   // gave up: reported
    }
    __syncthreads();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  };
  const int bv = a.v_bits, chunks = a.chunks;
  const TcStage geo = tc_stage(D, chunks, bv);
  const HeadLayout* L = a.layouts + int64_t(s) * a.n_kv + hk;
  const int ng = L->n_groups, nks = L->n_ksteps;

  // ---- staging of one tile's share of this wave, through registers: K records of the wave's
  // 16 tokens record-major ([token][chunk][16 B], unit u = token * chunks + chunk), group and
  // value norms [g][16] fp16 (value norms at g = kMaxGroups, planes of absent groups staged
  // too, so that no address depends on the layout), value segments of the wave's
  // D/4 coordinates.  Loads for the next tile are in flight while this tile is computed.
  const size_t reg = size_t(s) * a.n_kv + hk;
  const int64_t cap_tiles = a.capacity / kTile;
  const uint8_t* kc = a.k_codes + reg * cap_tiles * chunks * kTile * 16;
  const uint16_t* knp = a.k_norms + reg * cap_tiles * kMaxGroups * kTile;
  const uint8_t* vc = a.v_codes + reg * cap_tiles * D * 8 * bv;
  const uint16_t* vnp = a.v_norms + reg * cap_tiles * kTile;
  // Every lane loads and stores (no divergent memory operations): lanes past the last
  // 16-byte unit repeat the last unit, writing the same bytes to the same place.  A head
  // whose K budget is zero has no K records (chunks == 0): nothing is staged for K.
  const bool has_k = chunks > 0 && !win;
  uint32_t ksrc[MAXNK], kdst[MAXNK], vdst[MAXNV];
#pragma unroll
  for (int i = 0; i < MAXNK; ++i) {
    const int u = has_k ? min(64 * i + lane, 16 * chunks - 1) : 0;
    const int t = has_k ? u / chunks : 0, c = u - t * (has_k ? chunks : 1);
    ksrc[i] = uint32_t((c * kTile + 16 * wave + t) * 16);
    kdst[i] = uint32_t(16 * u);
  }
#pragma unroll
  for (int i = 0; i < MAXNV; ++i) vdst[i] = uint32_t(16 * min(64 * i + lane, D * bv / 8 - 1));
  const int nu = min(lane, 2 * kMaxGroups + 1);              // norm unit of this lane
  const bool nu_k = nu < 2 * kMaxGroups;                     // group norm (else value norm)
  const size_t nsrc = nu_k ? (size_t(nu >> 1) * kTile + 16 * wave + 8 * (nu & 1))
                           : (size_t(16 * wave + 8 * (nu & 1)));
  uint4 pk[MAXNK], pn, pv[MAXNV];
  auto load_tile = [&](int it) {
    const int tile = tbase + it * tstride;
    const uint8_t* kt = kc + size_t(tile) * chunks * kTile * 16;
    if (has_k) {
#pragma unroll
      for (int i = 0; i < MAXNK; ++i) pk[i] = *reinterpret_cast<const uint4*>(kt + ksrc[i]);
    }
    const uint16_t* nb = nu_k ? knp + size_t(tile) * kMaxGroups * kTile : vnp + size_t(tile) * kTile;
    pn = *reinterpret_cast<const uint4*>(nb + nsrc);
    const uint8_t* vt = vc + (size_t(tile) * D + CPW * wave) * 8 * bv;
#pragma unroll
    for (int i = 0; i < MAXNV; ++i) pv[i] = *reinterpret_cast<const uint4*>(vt + vdst[i]);
  };
  uint8_t* const buf = lds + kTcRing + wave * geo.bytes;
  auto store_tile = [&]() {
    if (has_k) {
#pragma unroll
      for (int i = 0; i < MAXNK; ++i) *reinterpret_cast<uint4*>(buf + kdst[i]) = pk[i];
    }
    *reinterpret_cast<uint4*>(buf + geo.n_off + 16 * nu) = pn;
#pragma unroll
    for (int i = 0; i < MAXNV; ++i) *reinterpret_cast<uint4*>(buf + geo.v_off + vdst[i]) = pv[i];
  };
  // ---- workgroup set-up and query prologue.  Global reads come in two rounds: everything
  // that does not depend on the layout descriptor (descriptor, level tables, query, first
  // tile), then the rotation rows.
  constexpr int NP = QShape<D>::NP, QI = QShape<D>::QI;
  constexpr int PW = (kPairWords + 255) / 256, SW = (kSingleHalves + 255) / 256;   // table pieces per thread
  static_assert(BGTQ_LAYOUT_BYTES == 256 * 16, "one 16-byte piece of the layout per thread");
  uint8_t* const pro = lds + kTcRing;             // aliases the ring, first written in the loop
  HeadLayout* const Ls = reinterpret_cast<HeadLayout*>(pro);
  float* const qc = reinterpret_cast<float*>(pro + BGTQ_LAYOUT_BYTES);           // q' [coordinate][8 heads]
  uint4* const qhi = reinterpret_cast<uint4*>(pro + tc_qhi_off(D));                // [k-step < 8][lane]
  uint4* const qlo = reinterpret_cast<uint4*>(lds + tc_qlo_off(D, chunks, bv));     // [k-step < 8][lane]
  uint4* const qlate = qlo + 64 * kQRegSteps;                                       // [k-step - 8][hi, lo][lane]
  f16x8 qh[kQRegSteps];
  {
    // a packed split's first tile depends on neither the length nor the layout: requested first
    if (!win) load_tile(0);
    const uint4 lw = reinterpret_cast<const uint4*>(L)[tid];
    uint2 pt[PW];
    uint32_t st[SW];
#pragma unroll
    for (int i = 0; i < PW; ++i)
      if (tid + 256 * i < kPairWords) pt[i] = c_pair_hl[tid + 256 * i];
#pragma unroll
    for (int i = 0; i < SW; ++i)
      if (tid + 256 * i < kSingleHalves) st[i] = c_single_hl[tid + 256 * i];
    float x0[QI], x1[QI];
    double fr = 0.0;
    {
      q_load<D, QT>(a, s, hk, tid, x0, x1);
      fr = a.rope_theta > 0.0 ? a.inv_freq[tid % NP] : 0.0;
    }
    if (win && count > 0) load_tile(0);
    reinterpret_cast<uint4*>(Ls)[tid] = lw;
    uint2* ptab = reinterpret_cast<uint2*>(lds);
#pragma unroll
    for (int i = 0; i < PW; ++i)
      if (tid + 256 * i < kPairWords) ptab[tid + 256 * i] = pt[i];
    uint32_t* stab = reinterpret_cast<uint32_t*>(lds + 8 * kPairWords);
#pragma unroll
    for (int i = 0; i < SW; ++i)
      if (tid + 256 * i < kSingleHalves) stab[tid + 256 * i] = st[i];
    uint32_t* pw = reinterpret_cast<uint32_t*>(lds + kTcP);
    for (int i = tid; i < 512; i += 256) {
      const int ln = (i >> 2) & 63;      // lane of the 16-byte B operand
      if ((ln & 15) >= 8) pw[i] = 0u;
    }
    {
      qops_zero(qhi, qlo, qlate, nks, tid);
      q_rope<D>(a, a.q_pos ? a.q_pos[s] : int64_t(len) - 1, fr, tid, x0, x1, qc);
    }
  }
  lds_barrier();
  const uint32_t wmask = wide_ksteps(Ls, nks, lane);
  const int nn = nks - __popc(wmask);               // narrow k-steps
  // per segment: x = byte offset of the window's first record dword, y = control of the
  // 4-bit-or-narrower decode (shift | 2w << 8 | pair table << 16; wider segments get a
  // harmless width-1 control), z = control of the any-width decode (shift | w << 8 | single
  // table << 16).
  // Segments past the last k-step, up to the register-resident ones, decode bit 0 at width 1.
  {
    uint4* kd = reinterpret_cast<uint4*>(lds + kTcDesc);
    const int nseg = 4 * (nks > kQRegSteps ? nks : kQRegSteps);
    for (int i = tid; i < nseg; i += 256) {
      const uint32_t seg = i < 4 * nks ? Ls->seg[i] : (1u << 16);
      const uint32_t o = seg & 0xffffu, w = (seg >> 16) & 15u;
      const uint32_t tbp = 8u * uint32_t(pair_base(int(w)));
      const uint32_t tbs = 8u * kPairWords + 4u * uint32_t(single_base(int(w)));
      const uint32_t fast = w <= 4 ? ((o & 31u) | ((2u * w) << 8) | (tbp << 16)) : (2u << 8);
      kd[i < 4 * nks ? 4 * kperm_of(wmask, nn, i >> 2) + (i & 3) : i] =
          uint4{4u * (o >> 5), fast, (o & 31u) | (w << 8) | (tbs << 16), 0u};
    }
    uint32_t* kn = reinterpret_cast<uint32_t*>(lds + kTcNorm);
    for (int i = tid; i < kMaxKSteps; i += 256) {
      const uint32_t kg = i < nks ? Ls->kgroups[i] : 0u;
      kn[i < nks ? kperm_of(wmask, nn, i) : i] = (32u * (kg & 0xffu)) | ((32u * ((kg >> 8) & 0xffu)) << 16);
    }
  }
  if (WIN && win) {
    // window role: B operand of k-step ks (coordinates 32 ks .. 32 ks + 31 in their original
    // order), lane (n, j): q'[head n][32 ks + 8 j + e] * softmax_scale * log2(e), fp16 high
    // part in registers and remainder in LDS; heads >= G and columns 8..15 are zero
    const float kscale = a.scale * kLog2e;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      f16x8 hi, lo;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = n < a.group ? qc[8 * (32 * ks + 8 * j + e) + n] * kscale : 0.0f;
        hi[e] = (_Float16)v;
        lo[e] = (_Float16)(v - float(hi[e]));
      }
      qh[ks] = hi;
      qlo[ks * 64 + lane] = __builtin_bit_cast(uint4, lo);
    }
  } else {
    if (a.givens) {
      qops_givens_rotate(a, Ls, qc, tid, 256);
      qops_scatter_rotated(a, Ls, qc, wmask, nn, tid, qhi, qlo, qlate);
    } else {
      qops_scatter<D>(a, Ls, qc, wmask, nn, tid, qhi, qlo, qlate);
    }
  }
  __syncthreads();   // also orders the prologue's reads of the ring before the first staging store

  // ---- query operands of the first k-steps in registers (zero past the last one)
  if (!win) {
#pragma unroll
    for (int ks = 0; ks < kQRegSteps; ++ks) {
      const uint4 z = uint4{0u, 0u, 0u, 0u};
      qh[ks] = __builtin_bit_cast(f16x8, ks < nks ? qhi[ks * 64 + lane] : z);
    }
    // the high parts sit in the ring's space: when some wave's staging reaches them, every
    // wave must hold its operands before the first staging store
    if (4 * geo.bytes > tc_qhi_off(D)) __syncthreads();
  }

  const uint4* kd = reinterpret_cast<const uint4*>(lds + kTcDesc);
  const uint32_t* knsel = reinterpret_cast<const uint32_t*>(lds + kTcNorm);
  const int nsh = n < 8 ? 0 : 16;
  const uint32_t krec = uint32_t(16 * chunks * n);
  const uint32_t knb = uint32_t(geo.n_off + 8 * j);
  const uint32_t wide = ((1u << nks) - 1u) & ~((1u << nn) - 1u);   // k-steps nn .. nks - 1
  // value windows: coordinate row 16 mi + n of the wave's block, tokens 32 st + 8 j ..
  const uint32_t vrow = uint32_t(geo.v_off + n * 8 * bv);
  const uint32_t vw0 = uint32_t(4 * ((8 * j * bv) >> 5)), vsh0 = uint32_t((8 * j * bv) & 31);
  const uint32_t vw1 = uint32_t(4 * (((32 + 8 * j) * bv) >> 5)), vsh1 = uint32_t(((32 + 8 * j) * bv) & 31);
  const uint32_t vtb = bv <= 5 ? 8u * uint32_t(pair_base(bv)) : 8u * kPairWords + 4u * uint32_t(single_base(bv));

  f32x4 acc[MTV];
#pragma unroll
  for (int mi = 0; mi < MTV; ++mi) acc[mi] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_part = 0.0f;
  const bool real_col = n < a.group;
  float* mx = reinterpret_cast<float*>(lds + kTcMx);   // [8 heads][4 waves][4 lane groups]

  // ---- softmax and P V of one tile from its logits S (rows: tokens 16 wave + 4 j + r, columns:
  // heads and the second group half); slots [vlo_t, valid) of the tile count (the window
  // role's first tile can start mid-tile; for the packed role vlo_t <= 0)
  auto finish_tile = [&](const f32x4& S, int tile, int valid, int vlo_t) {
    // ---- online softmax (base 2); head c = column c + column c + 8 (rotate the 16-lane row
    // by 8 with DPP); the tile maximum per head goes through LDS
    float v[4];
    float lm = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float sr = S[r];
      const float other = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, sr), 0x128, 0xf, 0xf, false));
      v[r] = sr + other;
      if (16 * wave + 4 * j + r >= valid || (WIN && 16 * wave + 4 * j + r < vlo_t)) v[r] = -INFINITY;
      lm = fmaxf(lm, v[r]);
    }
    if (a.logits && real_col) {
      float* lg = a.logits + (int64_t(s) * a.n_q + hk * a.group + n) * a.capacity + int64_t(tile) * kTile +
                  16 * wave + 4 * j;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (16 * wave + 4 * j + r < valid && (!WIN || 16 * wave + 4 * j + r >= vlo_t)) lg[r] = v[r] * kLn2;
    }
    if (n < 8) mx[16 * n + 4 * wave + j] = lm;
    lds_barrier();
    float tmax;
    {
      const float4* mr = reinterpret_cast<const float4*>(mx + 16 * (n & 7));
      const float4 m0 = mr[0], m1 = mr[1], m2 = mr[2], m3 = mr[3];
      tmax = fmaxf(fmaxf(fmaxf(fmaxf(m0.x, m0.y), fmaxf(m0.z, m0.w)), fmaxf(fmaxf(m1.x, m1.y), fmaxf(m1.z, m1.w))),
                   fmaxf(fmaxf(fmaxf(m2.x, m2.y), fmaxf(m2.z, m2.w)), fmaxf(fmaxf(m3.x, m3.y), fmaxf(m3.z, m3.w))));
    }
    const float m_new = fmaxf(m_run, tmax);          // finite: every tile has a valid token
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    const f16x4 vn = *reinterpret_cast<const f16x4*>(buf + geo.n_off + 32 * kMaxGroups + 8 * j);
    f16x4 bp;
    float psum = 0.0f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float p = __builtin_amdgcn_exp2f(v[r] - m_new);
      psum += p;
      bp[r] = (_Float16)(p * float(vn[r]));
    }
    l_part = l_part * alpha + psum;
    m_run = m_new;
    if (n < 8) {
      const int st = wave >> 1, jj = 2 * (wave & 1) + (j >> 1);
      *reinterpret_cast<f16x4*>(lds + kTcP + (st * 64 + jj * 16 + n) * 16 + 8 * (j & 1)) = bp;
    }
    if (__any(alpha != 1.0f)) {
#pragma unroll
      for (int mi = 0; mi < MTV; ++mi) acc[mi] *= alpha;
    }
    lds_barrier();

    // ---- P V for the wave's coordinates
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      if (32 * st < valid) {
        const f16x8 bpv = *reinterpret_cast<const f16x8*>(lds + kTcP + (st * 64 + lane) * 16);
        const uint32_t vw = st == 0 ? vw0 : vw1, vsh = st == 0 ? vsh0 : vsh1;
        uint32_t d0[MTV], d1[MTV], d2[MTV];
#pragma unroll
        for (int mi = 0; mi < MTV; ++mi) {
          const uint32_t ra = vrow + uint32_t(16 * mi * 8 * bv) + vw;
          d0[mi] = lds_u32(buf, ra);
          d1[mi] = lds_u32(buf, ra + 4);
          d2[mi] = bv > 4 ? lds_u32(buf, ra + 8) : 0u;
        }
#pragma unroll
        for (int mi = 0; mi < MTV; ++mi) {
          u32x4 vh, vl;
          decode8(d0[mi], d1[mi], d2[mi], int(vsh), bv, lds, vtb, vh, vl);
          acc[mi] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, vh), bpv, acc[mi], 0, 0, 0);
          acc[mi] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, vl), bpv, acc[mi], 0, 0, 0);
        }
      }
    }
  };

  // every load issued so far (query operands, set-up reads) is complete here, so the only
  // loads in flight inside the loop are the next tile's
  if (STEP && it_new == 0) {     // the first tile holds the new token: requested again after the append
    wait_append();
    load_tile(0);
  }
  __builtin_amdgcn_s_waitcnt(0);
  for (int it = 0; it < count; ++it) {
    const int tile = tbase + it * tstride;
    // tokens of this tile in the role's range: slots [vlo - 64 tile, valid)
    const int valid = vhi - tile * kTile < kTile ? vhi - tile * kTile : kTile;
    store_tile();                             // this wave's staging is read only by this wave
    asm volatile("" ::: "memory");            // issue the next tile's loads after these stores
    if (STEP && it + 1 == it_new) wait_append();
    if (it + 1 < count) load_tile(it + 1);

    f32x4 S = {0.f, 0.f, 0.f, 0.f};
    if (WIN && win) {
      // ---- window role: logits of tokens 16 wave + n from their fp16 keys (A rows; slots
      // outside the role's range read a valid slot and are masked).  The lane index is taken
      // afresh (opaque copy) so that no per-lane address of this branch is kept through the
      // loop.
      int wl = lane;
      asm volatile("" : "+v"(wl));
      const int tk = tile * kTile + 16 * wave + (wl & 15);
      const int tc = tk < vlo ? vlo : (tk >= vhi ? vhi - 1 : tk);
      const uint16_t* kr = a.k_window + (int64_t(reg) * a.window + tc % a.window) * D + 8 * (wl >> 4);
      constexpr int KB = D / 32 < 4 ? D / 32 : 4;     // k-steps whose keys are loaded together
#pragma unroll
      for (int k0 = 0; k0 < D / 32; k0 += KB) {
        uint4 kw[KB];
#pragma unroll
        for (int ks = 0; ks < KB; ++ks) kw[ks] = *reinterpret_cast<const uint4*>(kr + 32 * (k0 + ks));
#pragma unroll
        for (int ks = 0; ks < KB; ++ks) {
          const f16x8 A = __builtin_bit_cast(f16x8, kw[ks]);
          S = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, qh[k0 + ks], S, 0, 0, 0);
          S = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, __builtin_bit_cast(f16x8, qlo[(k0 + ks) * 64 + wl]), S, 0,
                                                     0, 0);
        }
      }
    } else {
      // ---- logits of tokens 16 wave + n (A rows).  Pass A issues a chunk's window reads and
      // level lookups (k-steps narrower than 5 bits), pass B runs the matrix cores on them;
      // wide k-steps are decoded separately afterwards.
      auto mfma_kstep = [&](const u32x4& raw, const u32x4& rawl, const f16x8& bh, const f16x8& bl, const f16x4& nv) {
        const f16x8 A = __builtin_bit_cast(f16x8, raw), Al = __builtin_bit_cast(f16x8, rawl);
        f32x4 T = {0.f, 0.f, 0.f, 0.f};
        T = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, bh, T, 0, 0, 0);
        T = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, bl, T, 0, 0, 0);
        T = __builtin_amdgcn_mfma_f32_16x16x32_f16(Al, bh, T, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) S[r] = fmaf(T[r], float(nv[r]), S[r]);
      };
      // narrow k-steps in chunks of 4, 2 and 2 (a chunk past the last narrow k-step is skipped;
      // inside the last one, slots past it are decoded but not multiplied)
      auto narrow_chunk = [&](auto kc_c, auto kn_c) {
        constexpr int kc = decltype(kc_c)::value, KC = decltype(kn_c)::value;
        {
          u32x4 raw[KC], rawl[KC];
          f16x4 nrm[KC];
          uint32_t wd0[KC], wd1[KC], ctl[KC];
#pragma unroll
          for (int q = 0; q < KC; ++q) {
            const uint2 d = *reinterpret_cast<const uint2*>(kd + 4 * (kc + q) + j);
            ctl[q] = d.y;
            wd0[q] = lds_u32(buf, krec + d.x);
            wd1[q] = lds_u32(buf, krec + d.x + 4);
            nrm[q] = *reinterpret_cast<const f16x4*>(buf + knb + ((knsel[kc + q] >> nsh) & 0xffffu));
          }
#pragma unroll
          for (int q = 0; q < KC; ++q) {
            const uint32_t x = __builtin_amdgcn_alignbit(wd1[q], wd0[q], ctl[q]);   // shift = ctl & 31
            const uint32_t w2 = ctl[q] >> 8;                                          // low 5 bits: 2w
            const uint32_t o4 = w2 << 1, o6 = w2 + o4, tb = ctl[q] >> 16;
            const uint32_t idx[4] = {__builtin_amdgcn_ubfe(x, 0u, w2), __builtin_amdgcn_ubfe(x, w2, w2),
                                     __builtin_amdgcn_ubfe(x, o4, w2), __builtin_amdgcn_ubfe(x, o6, w2)};
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) {
              const uint2 v = *reinterpret_cast<const uint2*>(lds + tb + 8 * idx[e2]);
              raw[q][e2] = v.x;
              rawl[q][e2] = v.y;
            }
          }
#pragma unroll
          for (int q = 0; q < KC; ++q)
            if (kc + q < nn)
              mfma_kstep(raw[q], rawl[q], qh[kc + q], __builtin_bit_cast(f16x8, qlo[(kc + q) * 64 + lane]), nrm[q]);
        }
      };
      static_assert(kQRegSteps == 8, "chunks 4 + 2 + 2");
      if (0 < nn) narrow_chunk(std::integral_constant<int, 0>{}, std::integral_constant<int, 4>{});
      if (4 < nn) narrow_chunk(std::integral_constant<int, 4>{}, std::integral_constant<int, 2>{});
      if (6 < nn) narrow_chunk(std::integral_constant<int, 6>{}, std::integral_constant<int, 2>{});
      // wide k-steps (codes of 5..8 bits in some segment): general decode
#pragma unroll
      for (int ks = 0; ks < kQRegSteps; ++ks) {
        if (wide & (1u << ks)) {
          const uint4 d = kd[4 * ks + j];
          const int w = int((d.z >> 8) & 15u);
          const uint32_t ka = krec + d.x;
          const uint32_t d0 = lds_u32(buf, ka), d1 = lds_u32(buf, ka + 4), d2 = lds_u32(buf, ka + 8);
          const f16x4 nv = *reinterpret_cast<const f16x4*>(buf + knb + ((knsel[ks] >> nsh) & 0xffffu));
          u32x4 ah, al;
          decode8_any(d0, d1, d2, int(d.z & 31u), w, lds, d.z >> 16, ah, al);
          mfma_kstep(ah, al, qh[ks], __builtin_bit_cast(f16x8, qlo[ks * 64 + lane]), nv);
        }
      }
      for (int ks = kQRegSteps; ks < nks; ++ks) {   // k-steps beyond the register-resident ones
        const uint4 d = kd[4 * ks + j];
        const int w = int((d.z >> 8) & 15u);
        const uint32_t ka = krec + d.x;
        const uint32_t d0 = lds_u32(buf, ka), d1 = lds_u32(buf, ka + 4), d2 = lds_u32(buf, ka + 8);
        const f16x4 nv = *reinterpret_cast<const f16x4*>(buf + knb + ((knsel[ks] >> nsh) & 0xffffu));
        u32x4 ah, al;
        decode8_any(d0, d1, d2, int(d.z & 31u), w, lds, d.z >> 16, ah, al);
        mfma_kstep(ah, al, __builtin_bit_cast(f16x8, qlate[(ks - kQRegSteps) * 128 + lane]),
                   __builtin_bit_cast(f16x8, qlate[(ks - kQRegSteps) * 128 + 64 + lane]), nv);
      }

    }
    finish_tile(S, tile, valid, WIN ? vlo - tile * kTile : 0);
  }

  // ---- partial result of this split: lane (n, j) holds head n, coordinates
  // D/4 wave + 16 mi + 4 j + r; the row sum is spread over lanes and waves.  The lane indices
  // are taken afresh here (opaque copies), so that no address of this epilogue is computed
  // before the tile loop and kept live through it.
  int le = lane;
  asm volatile("" : "+v"(le));
  const int ne = le & 15, je = le >> 4;
  float l = l_part;
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  float* lsm = mx + 128;
  if (je == 0 && ne < 8) lsm[8 * wave + ne] = l;
  __syncthreads();
  if (ne < a.group) {
    const int64_t row = (int64_t(s) * a.n_q + hk * a.group + ne) * a.n_split + split;
    float* dst = a.partial + row * D;
#pragma unroll
    for (int mi = 0; mi < MTV; ++mi)
      *reinterpret_cast<float4*>(dst + CPW * wave + 16 * mi + 4 * je) = float4{acc[mi][0], acc[mi][1], acc[mi][2], acc[mi][3]};
    if (wave == 0 && je == 0) a.part_ml[row] = float2{m_run, lsm[ne] + lsm[8 + ne] + lsm[16 + ne] + lsm[24 + ne]};
  }
}

#include "decode_stream.h"

// Merge the splits of one query head and undo the value rotation:
// out = R_v^T acc / (sqrt(d) * l), acc = sum_t p_t n_v,t C[code_t], from the per-split
// (m, l) pairs and accumulators; split i is weighted by exp2(m_i - max m).  Workgroup (h, s, q)
// of 256 threads first merges every coordinate of head h's splits: thread t takes coordinates
// 4 (t % (D/4)) .. + 3 of the splits t / (D/4) + NG k, in chunks of 16 requested together,
// rescaling its running sum when a chunk raises its maximum; the NG split groups are then
// combined through LDS, in group order.  Dense value rotation: the workgroup writes output
// coordinates 32 q .. 32 q + 31 (its R_v entries are requested before the split loads, so their
// latency overlaps the merge), as sums over 8 parts of the coordinates, in part order.  Givens
// layers mix every coordinate: one workgroup per head (q = 0) applies their transposes in
// reverse order.  Every output element is written once (no accumulation into out).
template <int D, bool GIV>
__global__ __launch_bounds__(256) void k_decode_combine(DecodeArgs a) {
  constexpr int NT = 256, C4 = D / 4, NG = NT / C4, CH = 16;   // CH splits per thread requested together
  constexpr int OQ = 32, KP = NT / OQ, KR = D / KP;    // outputs per workgroup, coordinate parts, rows per part
  static_assert(NT % C4 == 0 && NT >= D && NT >= D / 2, "thread roles of the merge");
  __shared__ float4 s_acc[NG][C4];
  __shared__ float2 s_ml[NG];
  __shared__ float s_x[D];
  __shared__ float s_part[KP][OQ];
  __shared__ float s_l;
  const int h = blockIdx.x, s = blockIdx.y, q = blockIdx.z;
  const int tid = threadIdx.x;
  const int ns = a.n_split;
  const size_t base = (size_t(s) * a.n_q + h) * ns;
  const float2* ml = a.part_ml + base;
  const float4* acc4 = reinterpret_cast<const float4*>(a.partial + base * D);
  const int c4 = tid % C4, g = tid / C4;
  // dense rotation: R_v[kp KR + k][32 q + t % 32] for this thread's part kp = t / 32
  const int ro = OQ * q + tid % OQ, kp = tid / OQ;
  float rv[GIV ? 1 : KR];
  if constexpr (!GIV) {
#pragma unroll
    for (int k = 0; k < KR; ++k) rv[k] = a.rot_v[size_t(kp * KR + k) * D + ro];
  }
  // structured rotation: pair slot t < D/2, layers from the last one (records fetched ahead)
  GivensSlot gs;
  gs.n = 0;
  if (GIV && tid < D / 2) {
    const uint4 hv = a.givens[D / 2 - 1];
    gs.n = min(int(hv.y), kMaxGivensLayers);
    gs.rec = a.givens + hv.x + (gs.n - 1) * (D / 2) + tid;
    gs.stride = -(D / 2);
#pragma unroll
    for (int l = 0; l < kGivensAhead; ++l) gs.fetch(l);
  }
  float4 v = {0.f, 0.f, 0.f, 0.f};
  float mr = -INFINITY, lr = 0.0f;
  for (int i0 = g; i0 < ns; i0 += NG * CH) {
    float4 x[CH];
    float2 mm[CH];
#pragma unroll
    for (int b = 0; b < CH; ++b) {
      const int i = i0 + NG * b;
      if (i < ns) {
        x[b] = acc4[size_t(i) * C4 + c4];
        mm[b] = ml[i];
      } else {
        x[b] = float4{0.f, 0.f, 0.f, 0.f};
        mm[b] = float2{-INFINITY, 0.f};
      }
    }
    float mc = mr;
#pragma unroll
    for (int b = 0; b < CH; ++b) mc = fmaxf(mc, mm[b].x);
    if (mc != -INFINITY) {
      const float sc = exp2f(mr - mc);               // 0 while nothing is summed yet
      v.x *= sc; v.y *= sc; v.z *= sc; v.w *= sc;
      lr *= sc;
#pragma unroll
      for (int b = 0; b < CH; ++b) {
        const float w = (mm[b].x == -INFINITY) ? 0.0f : exp2f(mm[b].x - mc);
        v.x = fmaf(w, x[b].x, v.x);
        v.y = fmaf(w, x[b].y, v.y);
        v.z = fmaf(w, x[b].z, v.z);
        v.w = fmaf(w, x[b].w, v.w);
        lr = fmaf(w, mm[b].y, lr);
      }
      mr = mc;
    }
  }
  s_acc[g][c4] = v;
  if (c4 == 0) s_ml[g] = float2{mr, lr};
  __syncthreads();
  if (tid < D) {                                     // coordinate tid over the split groups
    float mx = -INFINITY;
#pragma unroll
    for (int gg = 0; gg < NG; ++gg) mx = fmaxf(mx, s_ml[gg].x);
    float o = 0.0f, l = 0.0f;
#pragma unroll
    for (int gg = 0; gg < NG; ++gg) {
      const float w = (s_ml[gg].x == -INFINITY) ? 0.0f : exp2f(s_ml[gg].x - mx);
      o = fmaf(w, reinterpret_cast<const float*>(s_acc[gg])[tid], o);
      l = fmaf(w, s_ml[gg].y, l);
    }
    s_x[tid] = o;
    if (tid == 0) s_l = l;
  }
  __syncthreads();
  const float ltot = s_l;
  const float inv = (ltot > 0.0f) ? 1.0f / (ltot * sqrtf(float(D))) : 0.0f;
  float* const orow = a.out + (int64_t(s) * a.n_q + h) * D;
  if constexpr (GIV) {
    // the transpose, layers in reverse order, each pair as [[c, s], [-s, c]]
    const int nl = givens_count(a.givens, D);
#pragma unroll
    for (int i = 0; i < kMaxGivensLayers; ++i) {   // i-th layer from the last
      if (i < nl) {
        if (i < gs.n) {
          const int k = i % kGivensAhead;
          const int ia = int(gs.ab[k] & 0xffffu), ib = int(gs.ab[k] >> 16);
          const float xa = s_x[ia], xb = s_x[ib];
          s_x[ia] = fmaf(gs.c[k], xa, gs.s[k] * xb);
          s_x[ib] = fmaf(gs.c[k], xb, -gs.s[k] * xa);
          if (i + kGivensAhead < kMaxGivensLayers) gs.fetch(i + kGivensAhead);
        }
        __syncthreads();
      }
    }
    if (tid < D) orow[tid] = s_x[tid] * inv;
  } else {
    float o = 0.0f;
#pragma unroll
    for (int k = 0; k < KR; ++k) o = fmaf(rv[k], s_x[kp * KR + k], o);
    s_part[kp][tid % OQ] = o;
    __syncthreads();
    if (tid < OQ) {
      float t = s_part[0][tid];
#pragma unroll
      for (int p = 1; p < KP; ++p) t += s_part[p][tid];
      orow[OQ * q + tid] = t * inv;
    }
  }
  if (q == 0 && a.step && a.step_flag && h % a.group == 0 && tid == 0)   // ready for the next step
    a.step_flag[int64_t(s) * a.n_kv + h / a.group] = 0;
  if (q == 0 && a.step && h == 0 && tid == 0) {     // the decode step's length advance, after every reader
    const int len0 = a.lengths[s];
    if (len0 + 1 <= a.capacity) a.lengths[s] = len0 + 1;
  }
}

// the matrix-core kernel for a cache's record widths, query dtype and pass (a decode step, with
// its append role, or a decode call); with WIN, the window role is built in
template <int D, bool WIN>
auto mfma_kernel(bool narrow, bool bf16, bool step) -> void (*)(DecodeArgs, AppendArgs) {
  if (step)
    return narrow ? (bf16 ? k_decode_mfma<D, true, uint16_t, true, WIN> : k_decode_mfma<D, true, float, true, WIN>)
                  : (bf16 ? k_decode_mfma<D, false, uint16_t, true, WIN> : k_decode_mfma<D, false, float, true, WIN>);
  return narrow ? (bf16 ? k_decode_mfma<D, true, uint16_t, false, WIN> : k_decode_mfma<D, true, float, false, WIN>)
                : (bf16 ? k_decode_mfma<D, false, uint16_t, false, WIN> : k_decode_mfma<D, false, float, false, WIN>);
}

// a decode call, or (step != null, matrix-core path) a decode step: one more workgroup per
// (sequence, KV head), the append role, ahead of the splits
template <int D>
hipError_t launch_decode_d(const DecodeArgs& a, bgtq_dtype q_dt, hipStream_t st, const AppendArgs* step = nullptr) {
  const dim3 grid(a.n_split + (step ? 1 : 0), a.n_kv, a.batch);
  if (a.use_stream) {
    if constexpr (D <= 128) {
      const bool bf16 = q_dt == BGTQ_BF16;
      // batch launches of several rounds start the longest sequences first
      const bool order = a.stream_whole_tiles != 0 && a.batch <= kLptMaxBatch;
      void (*fn)(DecodeArgs, AppendArgs) =
          order ? (step ? (bf16 ? k_decode_stream<D, uint16_t, true, true> : k_decode_stream<D, float, true, true>)
                        : (bf16 ? k_decode_stream<D, uint16_t, false, true> : k_decode_stream<D, float, false, true>))
                : (step ? (bf16 ? k_decode_stream<D, uint16_t, true, false> : k_decode_stream<D, float, true, false>)
                        : (bf16 ? k_decode_stream<D, uint16_t, false, false> : k_decode_stream<D, float, false, false>));
      hipLaunchKernelGGL(fn, grid, dim3(kStreamThreads), 0, st, a, step ? *step : AppendArgs{});
    } else {
      return hipErrorInvalidValue;
    }
  } else if (a.use_mfma) {
    int lds = tc_lds_bytes(D, a.chunks, a.v_bits);
    if (step && lds < int(kStepAppendLds)) lds = int(kStepAppendLds);
    const bool narrow = a.chunks <= 4 && a.v_bits <= 4, bf16 = q_dt == BGTQ_BF16;
    void (*fn)(DecodeArgs, AppendArgs) = a.window > 0 ? mfma_kernel<D, true>(narrow, bf16, step != nullptr)
                                                      : mfma_kernel<D, false>(narrow, bf16, step != nullptr);
    if (lds > 64 * 1024) {
      const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, lds);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(fn, grid, dim3(256), size_t(lds), st, a, step ? *step : AppendArgs{});
  } else {
    if (q_dt == BGTQ_BF16)
      hipLaunchKernelGGL(k_decode_prep<uint16_t>, dim3(a.n_kv, a.batch, kPrepZ), dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL(k_decode_prep<float>, dim3(a.n_kv, a.batch, kPrepZ), dim3(256), 0, st, a);
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
  if (a.givens) hipLaunchKernelGGL((k_decode_combine<D, true>), dim3(a.n_q, a.batch, 1), dim3(256), 0, st, a);
  else hipLaunchKernelGGL((k_decode_combine<D, false>), dim3(a.n_q, a.batch, D / 32), dim3(256), 0, st, a);
  return hipGetLastError();
}


}  // namespace

// ===================================================================== launchers

hipError_t launch_decode_step(const AppendArgs& aa, const DecodeArgs& da, bgtq_dtype kv_dt, bgtq_dtype q_dt,
                              hipStream_t st) {
  AppendArgs a2 = aa;
  a2.kv_bf16 = kv_dt == BGTQ_BF16;
  switch (da.d) {
    case 64: return launch_decode_d<64>(da, q_dt, st, &a2);
    case 128: return launch_decode_d<128>(da, q_dt, st, &a2);
    case 256: return launch_decode_d<256>(da, q_dt, st, &a2);
    default: return hipErrorInvalidValue;
  }
}

size_t decode_step_bytes(int batch, int n_kv_heads) { return size_t(batch) * n_kv_heads * 4; }

namespace {
// Workspace of the allocation-free decode step: one array per GPU, part of the code object.
// Host code must not pass the array's name to a kernel (on the host it is only a stand-in);
// scratch_address gives the device address to use instead.
__device__ __align__(256) uint8_t scratch[BGTQ_NOALLOC_SCRATCH_BYTES];

__global__ __launch_bounds__(256) void k_clear_flags(int32_t* __restrict__ flags, int n) {
  const int i = int(blockIdx.x) * 256 + int(threadIdx.x);
  if (i < n) flags[i] = 0;
}
}  // namespace

hipError_t scratch_address(void** ptr) { return hipGetSymbolAddress(ptr, HIP_SYMBOL(scratch)); }

hipError_t launch_clear_flags(int32_t* flags, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_clear_flags, dim3((n + 255) / 256), dim3(256), 0, s, flags, n);
  return hipGetLastError();
}

hipError_t upload_tables(const Tables& t) {
  hipError_t e = hipMemcpyToSymbol(HIP_SYMBOL(c_thr), t.thr, sizeof(t.thr));
  if (e == hipSuccess) e = hipMemcpyToSymbol(HIP_SYMBOL(c_cen), t.cen, sizeof(t.cen));
  if (e == hipSuccess) e = hipMemcpyToSymbol(HIP_SYMBOL(c_dgain), t.dgain, sizeof(t.dgain));
  if (e == hipSuccess) e = hipMemcpyToSymbol(HIP_SYMBOL(c_pair), t.pair, sizeof(t.pair));
  if (e == hipSuccess) e = hipMemcpyToSymbol(HIP_SYMBOL(c_single), t.single, sizeof(t.single));
  if (e == hipSuccess) e = hipMemcpyToSymbol(HIP_SYMBOL(c_pair_hl), t.pair_hl, sizeof(t.pair_hl));
  if (e == hipSuccess) e = hipMemcpyToSymbol(HIP_SYMBOL(c_single_hl), t.single_hl, sizeof(t.single_hl));
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

hipError_t launch_prefill_alloc(const void* keys, bgtq_dtype dt, int n_heads, int64_t n_tokens, int d, int64_t sh,
                               int64_t st, int pairing, double* partial, int increments, int b_min, int b_max,
                               double* energy_out, uint8_t* widths, HeadLayout* layouts, hipStream_t s) {
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
  hipLaunchKernelGGL(k_energy_allocate, dim3(n_heads), dim3(64), 0, s, partial, n_chunks, n_tokens, n, increments,
                     b_min, b_max, pairing, energy_out, widths, layouts);
  return hipGetLastError();
}

hipError_t launch_allocate(const double* energy, int n_heads, int n_blocks, int increments, int b_min,
                           int b_max, int pairing, uint8_t* widths, HeadLayout* layouts, hipStream_t s) {
  hipLaunchKernelGGL(k_allocate, dim3(n_heads), dim3(64), 0, s, energy, n_blocks, increments, b_min, b_max,
                     pairing, widths, layouts);
  return hipGetLastError();
}

namespace {
// the one-token append kernel for the input dtype, value staging and window
template <bool WIN, bool GIV>
auto append_one_kernel(bool bf16, bool stage_v) -> void (*)(AppendArgs) {
  return bf16 ? (stage_v ? k_append_one<uint16_t, true, WIN, GIV> : k_append_one<uint16_t, false, WIN, GIV>)
              : (stage_v ? k_append_one<float, true, WIN, GIV> : k_append_one<float, false, WIN, GIV>);
}
}  // namespace

// k_append for head dims up to DM, the input dtype and the rotation kind
template <int DM>
hipError_t launch_append_many(const AppendArgs& a, bgtq_dtype dt, dim3 grid, hipStream_t s) {
  const bool bf = dt == BGTQ_BF16;
  void (*fn)(AppendArgs) = a.givens ? (bf ? k_append<uint16_t, DM, true> : k_append<float, DM, true>)
                                    : (bf ? k_append<uint16_t, DM, false> : k_append<float, DM, false>);
  const size_t lds = append_lds_bytes(a.d, DM);
  if (lds > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(fn, grid, dim3(256), lds, s, a);
  return hipSuccess;
}

hipError_t launch_append(const AppendArgs& a, bgtq_dtype dt, int n_seqs, hipStream_t s) {
  if (a.n_new == 1) {   // one token per sequence: one workgroup per (sequence, KV head)
    const bool stage_v = a.d <= 128;
    const size_t lds = append_one_lds_bytes(a.d, stage_v, stage_v && !a.givens);
    const bool bf = dt == BGTQ_BF16, w = a.window > 0;
    void (*fn)(AppendArgs) = a.givens ? (w ? append_one_kernel<true, true>(bf, stage_v) : append_one_kernel<false, true>(bf, stage_v))
                                      : (w ? append_one_kernel<true, false>(bf, stage_v) : append_one_kernel<false, false>(bf, stage_v));
    const hipError_t e =
        hipFuncSetAttribute(reinterpret_cast<const void*>(fn), hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(fn, dim3(n_seqs * a.n_kv_heads), dim3(1024), lds, s, a);
    if (a.advance)
      hipLaunchKernelGGL(k_advance, dim3((n_seqs + 63) / 64), dim3(64), 0, s, a.lengths, a.seq_begin, n_seqs,
                         a.n_new, a.capacity);
    return hipGetLastError();
  }
  const int halves = int((a.n_new + kHalf - 1) / kHalf) + 1;
  const dim3 grid(halves, a.n_kv_heads, n_seqs);
  const hipError_t e = a.d <= 64 ? launch_append_many<64>(a, dt, grid, s)
                       : a.d <= 128 ? launch_append_many<128>(a, dt, grid, s)
                                    : launch_append_many<256>(a, dt, grid, s);
  if (e != hipSuccess) return e;
  if (a.window > 0) {
    const int64_t m = a.n_new < a.window ? a.n_new : a.window;
    const dim3 wgrid(unsigned((m * a.d + 255) / 256), a.n_kv_heads, n_seqs);
    if (dt == BGTQ_BF16)
      hipLaunchKernelGGL(k_window_store<uint16_t>, wgrid, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL(k_window_store<float>, wgrid, dim3(256), 0, s, a);
  }
  hipLaunchKernelGGL(k_advance, dim3((n_seqs + 63) / 64), dim3(64), 0, s, a.lengths, a.seq_begin, n_seqs, a.n_new,
                     a.capacity);
  return hipGetLastError();
}

// Transposed copies of the rotation bank (block m = 2 blockIdx.y + 2) and of the value rotation
// (blockIdx.y = d / 2).
__global__ __launch_bounds__(256) void k_transpose_rotations(const float* __restrict__ bank, const float* __restrict__ rv,
                                                             int d, float* __restrict__ bank_t, float* __restrict__ rv_t) {
  const bool value = int(blockIdx.y) == d / 2;
  const int m = value ? d : 2 * int(blockIdx.y) + 2;
  const float* src = value ? rv : bank + bank_offset(m);
  float* dst = value ? rv_t : bank_t + bank_offset(m);
  for (int e = int(blockIdx.x) * 256 + int(threadIdx.x); e < m * m; e += int(gridDim.x) * 256) {
    const int row = e / m, col = e - row * m;
    dst[col * m + row] = src[e];
  }
}

hipError_t launch_transpose_rotations(const float* rot_bank, const float* rot_v, int d, float* rot_bank_t,
                                      float* rot_v_t, hipStream_t s) {
  hipLaunchKernelGGL(k_transpose_rotations, dim3((d * d + 255) / 256, d / 2 + 1), dim3(256), 0, s, rot_bank, rot_v,
                     d, rot_bank_t, rot_v_t);
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
  // matrix-core kernel: four resident workgroups on each of the 256 compute units, tile
  // ranges balanced to within one tile; vector-ALU kernel: about 1024 workgroups
  const int64_t target = 1024;
  int64_t want = (target + units - 1) / units;
  const int64_t per_split = mfma ? 4 : 8;             // tiles per split at least
  const int64_t by_work = (tiles + per_split - 1) / per_split;
  if (want > by_work) want = by_work;
  if (want < 1) want = 1;
  if (want > 1024) want = 1024;
  return int(want);
}

bool decode_stream_fits(int d, int chunks, int v_bits) { return stream_fits(d, chunks, v_bits); }

int decode_stream_splits(int batch, int n_kv_heads) {
  // Few (sequence, KV head) units: one workgroup per compute unit, 256 over the units, one of
  // each unit's share left to a decode step's append role.  A batch of many units: the
  // sequences' lengths may differ widely while every unit takes the same number of splits, so
  // the grid is two rounds of the compute units, the longest sequences' workgroups first (the
  // pass maps grid slots to sequences by length), and the dispatcher hands a freed compute unit
  // the next workgroup: the second round's short workgroups fill in behind the long ones.  (Four
  // rounds pay the pass's fixed cost per workgroup twice as often.)
  const int64_t units = int64_t(batch) * n_kv_heads;
  if (batch > 1 && units >= 16) {
    const int64_t over = 2 * 256 / units;
    return over > 2 ? int(over) : 2;
  }
  const int64_t base = 256 / units;
  return base > 2 ? int(base - 1) : 1;
}

bool decode_stream_whole_tiles(int batch, int n_kv_heads) {
  return batch > 1 && int64_t(batch) * n_kv_heads >= 16;   // the oversubscribed grid above
}

size_t decode_qrot_bytes(int batch, int n_kv_heads, int d) {
  return size_t(batch) * n_kv_heads * d * kQPad * 4;
}

}  // namespace bgtq
