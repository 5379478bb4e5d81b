// Key-only logit-error diagnostic for gfx950 (CDNA4, wave64).
//
// Method: "RoPE-Aware Bit Allocation for KV-Cache Quantization" (arXiv 2606.24033), abstract:
// Block-GTQ is judged by how well it keeps the RoPE query-key logits, measured per layer as
// the mean absolute error of those logits when only the keys are quantized, at 2 and 3 bits
// per coordinate, against uniform TQ-MSE at the same budget.
//
// Given the logits a decode over a quantized cache produced (fp32, [batch][n_q][capacity]),
// this pass forms the exact logits from the unquantized post-RoPE keys and reduces
// |quantized - exact| per (sequence, query head).  The exact logits are a dense contraction,
// Q' [16 heads x d] . K^T [d x tokens], so they run on the fp32 matrix cores
// (v_mfma_f32_16x16x4_f32: full fp32 products and sums), 16 tokens per instruction block.

#include <hip/hip_runtime.h>

#include "bgtq_internal.h"

namespace bgtq {
namespace {

constexpr double kTwoPiD = 6.283185307179586476925286766559;
constexpr int kStrip = 16;                       // tokens per matrix-core block
constexpr int kStripsPerWave = kErrChunk / kStrip / 4;

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float ld1(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float ld1(const uint16_t* p, int64_t i) { return __uint_as_float(uint32_t(p[i]) << 16); }

// four consecutive coordinates (16-byte aligned for fp32, 8-byte for bf16)
__device__ __forceinline__ float4 ld4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ float4 ld4(const uint16_t* p) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  return float4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
                __uint_as_float(u.y & 0xffff0000u)};
}

// Workgroup = (chunk of kErrChunk tokens, KV head, sequence); 4 waves, wave w takes the
// 16-token strips w, w + 4, w + 8, w + 12 of the chunk.  In a strip, lane l holds token
// t0 + l % 16 and the coordinates 16 i + 4 (l / 16) + e (i < D/16, e < 4) in registers;
// k-step (i, e) feeds the matrix core that coordinate of the 16 tokens (A) and of the 16
// rotated queries (B), so the D/4 k-steps cover every coordinate once.  Lane l then holds
// the exact logits of head l % 16 at tokens t0 + 4 (l / 16) + r.  The first strip's keys
// and logits are loaded before the query rotation.  One strip in flight per wave keeps the
// kernel near 100 registers and five waves per SIMD, which measured faster than two or four
// strips per wave (fewer waves) or a prefetch of the next strip.
template <int D, typename KT, typename QT>
__global__ __launch_bounds__(256) void k_logit_err(LogitErrArgs a) {
  constexpr int NP = D / 2, QS = D + 4;          // padded rows of q'
  constexpr int S = 1;                           // strips in flight per wave (more cost occupancy)
  constexpr int KI = D / 16;                     // float4 of a lane's key share
  __shared__ __attribute__((aligned(16))) float qs[16 * QS];
  __shared__ double red[4][16];
  const int chunk = blockIdx.x, hk = blockIdx.y, s = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = a.group;
  const int64_t len = a.lengths[s] < a.capacity ? int64_t(a.lengths[s]) : a.capacity;
  const int64_t tb = int64_t(chunk) * kErrChunk;
  double* part = a.partial + (int64_t(s) * a.n_q + int64_t(hk) * G) * a.n_chunk + chunk;
  if (tb >= len) {                               // the whole workgroup leaves together
    if (tid < G) part[int64_t(tid) * a.n_chunk] = 0.0;
    return;
  }
  const int n = lane & 15, g = lane >> 4;
  const KT* kbase = static_cast<const KT*>(a.keys) + int64_t(s) * a.stride_seq + int64_t(hk) * a.stride_head;
  const float* lrow = a.logits + (int64_t(s) * a.n_q + int64_t(hk) * G + (n < G ? n : 0)) * a.capacity;
  const double sc = a.scale;
  double err = 0.0;
  float4 k[S][KI];
  float lq[S][4];
  // keys and quantized logits of strips sg .. sg + S - 1 (zero past the length)
  auto load_group = [&](int sg) {
#pragma unroll
    for (int u = 0; u < S; ++u) {
      const int64_t t0 = tb + int64_t(kStrip) * (wave + 4 * (sg + u));
      const int64_t t = t0 + n;
      if (t < len) {
        const KT* kr = kbase + t * a.stride_token + 4 * g;
#pragma unroll
        for (int i = 0; i < KI; ++i) k[u][i] = ld4(kr + 16 * i);
      } else {
#pragma unroll
        for (int i = 0; i < KI; ++i) k[u][i] = float4{0.0f, 0.0f, 0.0f, 0.0f};
      }
      const int64_t tr = t0 + 4 * g;
      if (tr + 3 < len) {
        const float4 v = *reinterpret_cast<const float4*>(lrow + tr);
        lq[u][0] = v.x, lq[u][1] = v.y, lq[u][2] = v.z, lq[u][3] = v.w;
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) lq[u][r] = tr + r < len ? lrow[tr + r] : 0.0f;
      }
    }
  };
  load_group(0);
  {
    // q' = RoPE(q, pos) of the group's heads (angle formed and reduced modulo 2 pi in fp64,
    // then fp32 sine and cosine); rows >= G zero.  Overlaps the first loads.
    const int64_t pos = a.q_pos ? a.q_pos[s] : len - 1;
    const QT* q = static_cast<const QT*>(a.q) + (int64_t(s) * a.n_q + int64_t(hk) * G) * D;
    for (int idx = tid; idx < 16 * NP; idx += 256) {
      const int h = idx / NP, j = idx - h * NP;
      const int ca = a.pairing ? 2 * j : j, cb = a.pairing ? 2 * j + 1 : j + NP;
      float ra = 0.0f, rb = 0.0f;
      if (h < G) {
        const float x0 = ld1(q + int64_t(h) * D, ca), x1 = ld1(q + int64_t(h) * D, cb);
        float sv = 0.0f, cv = 1.0f;
        if (a.rope_theta > 0.0) {
          const double ang = double(pos) * a.inv_freq[j];
          sincosf(float(ang - kTwoPiD * floor(ang * (1.0 / kTwoPiD))), &sv, &cv);
        }
        ra = x0 * cv - x1 * sv;
        rb = x0 * sv + x1 * cv;
      }
      qs[h * QS + ca] = ra;
      qs[h * QS + cb] = rb;
    }
  }
  __syncthreads();
#pragma unroll 1
  for (int sg = 0;;) {
    if (tb + int64_t(kStrip) * (wave + 4 * sg) >= len) break;   // wave-uniform
    f32x4 acc[S];
#pragma unroll
    for (int u = 0; u < S; ++u) acc[u] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      const float4 b = *reinterpret_cast<const float4*>(qs + n * QS + 16 * i + 4 * g);
#pragma unroll
      for (int u = 0; u < S; ++u) acc[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(k[u][i].x, b.x, acc[u], 0, 0, 0);
#pragma unroll
      for (int u = 0; u < S; ++u) acc[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(k[u][i].y, b.y, acc[u], 0, 0, 0);
#pragma unroll
      for (int u = 0; u < S; ++u) acc[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(k[u][i].z, b.z, acc[u], 0, 0, 0);
#pragma unroll
      for (int u = 0; u < S; ++u) acc[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(k[u][i].w, b.w, acc[u], 0, 0, 0);
    }
    if (n < G) {
#pragma unroll
      for (int u = 0; u < S; ++u) {
        const int64_t tr = tb + int64_t(kStrip) * (wave + 4 * (sg + u)) + 4 * g;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (tr + r < len) err += fabs(double(lq[u][r]) - sc * double(acc[u][r]));
      }
    }
    sg += S;
    if (sg >= kStripsPerWave) break;
    load_group(sg);
  }
  // lanes n, n + 16, n + 32, n + 48 hold head n; fixed reduction order
  err += __shfl_xor(err, 16);
  err += __shfl_xor(err, 32);
  if (lane < 16) red[wave][lane] = err;
  __syncthreads();
  if (tid < G) part[int64_t(tid) * a.n_chunk] = ((red[0][tid] + red[1][tid]) + red[2][tid]) + red[3][tid];
}

// One wave per (sequence, query head): the chunk sums in a fixed order, then the mean.
__global__ __launch_bounds__(64) void k_logit_err_final(LogitErrArgs a) {
  const int h = blockIdx.x, s = blockIdx.y, lane = threadIdx.x;
  const double* part = a.partial + (int64_t(s) * a.n_q + h) * a.n_chunk;
  double acc = 0.0;
#pragma unroll 8
  for (int c = lane; c < a.n_chunk; c += 64) acc += part[c];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
  if (lane == 0) {
    const int64_t len = a.lengths[s] < a.capacity ? int64_t(a.lengths[s]) : a.capacity;
    a.mae[int64_t(s) * a.n_q + h] = len > 0 ? acc / double(len) : 0.0;
  }
}

template <int D, typename KT>
hipError_t launch_err_d(const LogitErrArgs& a, bgtq_dtype q_dt, hipStream_t st) {
  const dim3 grid(a.n_chunk, a.n_kv, a.batch);
  if (q_dt == BGTQ_BF16)
    hipLaunchKernelGGL((k_logit_err<D, KT, uint16_t>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((k_logit_err<D, KT, float>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_err_k(const LogitErrArgs& a, bgtq_dtype k_dt, bgtq_dtype q_dt, hipStream_t st) {
  return k_dt == BGTQ_BF16 ? launch_err_d<D, uint16_t>(a, q_dt, st) : launch_err_d<D, float>(a, q_dt, st);
}

}  // namespace

hipError_t launch_logit_error(const LogitErrArgs& a, bgtq_dtype k_dt, bgtq_dtype q_dt, hipStream_t st) {
  hipError_t e = hipSuccess;
  switch (a.d) {
    case 64: e = launch_err_k<64>(a, k_dt, q_dt, st); break;
    case 128: e = launch_err_k<128>(a, k_dt, q_dt, st); break;
    case 256: e = launch_err_k<256>(a, k_dt, q_dt, st); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_logit_err_final, dim3(a.n_q, a.batch), dim3(64), 0, st, a);
  return hipGetLastError();
}

}  // namespace bgtq
