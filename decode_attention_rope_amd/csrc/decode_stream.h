// Streamed split pass of the matrix-core decode (included by kernels.hip, inside its
// anonymous namespace, after the query prologue helpers and the decode step's append role).
//
// RoPE query-key logits over the packed cache, softmax and the value sum (abstract: the
// logit is a sum of per-block 2-D RoPE terms; the serving path attends over a packed K3V3
// cache at 128K context).  One workgroup of 8 waves per split.  The W = 8 n_split waves of a
// (sequence, KV head) take its tiles round-robin (wave v: tiles v, v + W, ...), then the
// remaining tiles as quarters (one 16-token row block each), one per wave in the same order.  Every wave works on its
// own units: it stages a unit's tile with direct-to-LDS loads into its own LDS slot (the next
// unit's loads are in flight meanwhile), computes the logits, runs its own online softmax and
// accumulates P V; no workgroup barrier falls inside the unit loop.  The 8 waves' results are
// merged once, at the end, into the split's partial result (the format k_decode_combine reads).
//
//   logits  per k-step ks (32 storage positions of at most two width groups) and row block
//           (16 tokens): lane (n, j) decodes the 8 codes of its token's segment (ks, j) into
//           fp16 level pairs hi + lo; two MFMA operands per row block hold codes 0..3 and
//           4..7 with interleaved k slots (hi 0, hi 1, lo 0, lo 1, ...), B repeats the rotated
//           query's halves to match (columns 0-7: the G heads restricted to the k-step's first
//           width group, columns 8-15: its second), in high part and remainder; four
//           v_mfma_f32_16x16x32_f16 give T, then S += T * n_group.  Row r of row block rb is
//           token 32 (rb / 2) + 8 (r / 4) + 4 (rb % 2) + r % 4 of the tile, so that lane (c, j)
//           ends up holding tokens 8 j .. 8 j + 7 of each 32-token block: exactly the k slots
//           of the P V operand below, with no exchange.
//   values  A = the fp16 value levels of 16 rotated coordinates x 8 tokens per lane group (k slot
//           e = token 32 b + 8 j + e), B = P n_v in fp16 from the softmax registers, one MFMA per
//           M-tile and 32-token value block; acc holds 16 coordinates x 16 columns per M-tile.
// For the keys the hi + lo split carries the fp32 Lloyd-Max levels to about 2^-22 relative.

constexpr int kStreamWaves = 8;
constexpr int kStreamThreads = 64 * kStreamWaves;

// One tile's staging slot in LDS (bytes): K records token-major [64][16 chunks], the K norm
// planes [8][64] fp16 (those of the layout's groups filled), the value norms [64] fp16, the
// value codes [D][8 b_v] (coordinate-major, as in HBM), 16 bytes of slack for window reads past
// the end.  A tile arrives with
// `chunks` + 1 + v_loads direct loads of 1 KiB per wave (the last value load partial).
struct StreamSlot {
  int kn_off, vn_off, vc_off, bytes;
  int v_units, v_loads;              // 16-byte value units (norms first) and their loads
};
__host__ __device__ inline StreamSlot stream_slot(int D, int chunks, int bv) {
  StreamSlot g;
  g.kn_off = 1024 * chunks;
  g.vn_off = g.kn_off + 2 * kMaxGroups * kTile;
  g.vc_off = g.vn_off + 2 * kTile;
  g.bytes = g.vc_off + D * 8 * bv + 16;
  g.v_units = 8 + D * bv / 2;
  g.v_loads = (g.v_units + 63) / 64;
  return g;
}
// Static LDS of the pass: two staging rings of one slot per wave (separate objects, so that the
// compiler's waits for one ring's loads leave the other's in flight), decoder tables, k-step
// descriptors, the prologue's area (layout copy, q', B operands), the merge's exchange.
__host__ __device__ constexpr int stream_slot_max(int D) { return D == 128 ? 7424 : 5376; }

// Batch launches of several workgroup rounds: the dispatcher starts workgroups in index order,
// so grid slot z takes the z-th longest sequence (equal lengths in index order).  The longest
// sequences' workgroups then start first and the last round holds short ones (longest
// processing time first).  The ranks come from the lengths every workgroup reads alike, so the
// slots map one to one onto the sequences, and a decode step's append role (workgroup 0 of a
// slot) still starts before the splits that wait for it.  Batches of more than kLptMaxBatch
// sequences keep index order (the launch picks the instantiation).  lds: kLptMaxBatch + 1 ints.
constexpr int kLptMaxBatch = 64;
__device__ __forceinline__ int seq_longest_first(const int32_t* lengths, int nb, int* lds) {
  const int t = threadIdx.x;
  if (t < nb) lds[t] = lengths[t];
  __syncthreads();
  if (t < nb) {
    const int lt = lds[t];
    int rank = 0;
    for (int u = 0; u < nb; ++u) {
      const int lu = lds[u];
      rank += (lu > lt || (lu == lt && u < t)) ? 1 : 0;
    }
    if (rank == int(blockIdx.z)) lds[kLptMaxBatch] = t;
  }
  __syncthreads();
  return __builtin_amdgcn_readfirstlane(lds[kLptMaxBatch]);
}
constexpr int kSTabPair = 0;                                   // uint2 [kPairWords] hi, lo
constexpr int kSTabSingle = kSTabPair + 8 * kPairWords;        // uint32 [kSingleHalves] hi | lo << 16
constexpr int kSTabV = kSTabSingle + 4 * kSingleHalves;       // uint32 [84] high-part pairs of widths 1..3
constexpr int kVPairWords = 84;                                 // 4 + 16 + 64 entries
constexpr int kSTabVQ = kSTabV + 4 * kVPairWords;             // uint2 [272] fp16 levels of 4 codes, widths 1, 2
constexpr int kVQuadWords = 16 + 256;
constexpr int kSTabBytes = (kSTabVQ + 8 * kVQuadWords + 255) & ~255;
__host__ __device__ constexpr int stream_pro_bytes(int D) {
  return BGTQ_LAYOUT_BYTES + 32 * D + 2 * 1024 * kQRegSteps;   // layout, q' [D][8], B hi [8][64], B lo [8][64]
}
// whether the streamed pass serves a cache: head dims 64 and 128 without a window, K records of
// at most 4 chunks, tiles that fit a ring slot
__host__ __device__ inline bool stream_fits(int D, int chunks, int bv) {
  return (D == 64 || D == 128) && chunks <= 4 && stream_slot(D, chunks, bv).bytes <= stream_slot_max(D);
}

// the window of a segment: bits [sh, sh + 32) of d1:d0 as one dword
__device__ __forceinline__ uint32_t win32(uint32_t d0, uint32_t d1, uint32_t sh) {
  return __builtin_amdgcn_alignbit(d1, d0, sh);
}

// x as an opaque wave-uniform value: the compiler keeps it in a register from here on instead
// of reading the kernel argument again where it is used (a late re-read of the argument
// segment costs a memory round trip after the tile loop)
template <typename T>
__device__ __forceinline__ T keep_s(T x) {
  asm volatile("" : "+s"(x));
  return x;
}
// the same for a global-memory pointer, returned in the global address space (an opaque generic
// pointer would make its accesses flat ones, which later LDS waits also wait for)
template <typename T>
using gptr = __attribute__((address_space(1))) T*;
template <typename T>
__device__ __forceinline__ gptr<T> keep_g(T* p) {
  asm volatile("" : "+s"(p));
  return (gptr<T>)p;
}

// 16 bytes per lane from global address p to LDS at lds + 16 lane (lds the same for the whole
// wave) as one direct-to-LDS load.  It is issued from asm so that the compiler's wait insertion
// does not track it: that pass cannot tell the two staging rings apart and would make every LDS
// read of the tile loop wait for every staging load in flight, including the next tile's.  The
// waits for these loads are therefore explicit (vmcnt, which counts vector memory operations in
// issue order).  M0 holds the LDS address for the load and is restored afterwards.
__device__ __forceinline__ void stage16(const void* p, const void* lds) {
  const uint32_t l = __builtin_amdgcn_readfirstlane(uint32_t(reinterpret_cast<uintptr_t>(lds)));
  uint32_t keep;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(keep)
      : "s"(l), "v"(p)
      : "memory");
}

// Matrix-core operands of eight decoded codes, k slots interleaved: A1 holds the levels of codes
// 0..3 as (hi 0, hi 1, lo 0, lo 1, hi 2, hi 3, lo 2, lo 3), A2 those of codes 4..7, so that each
// pair lookup (hi pair, lo pair) lands in its operand as loaded.  The matching B operand repeats
// the other factor: (x 0, x 1, x 0, x 1, x 2, x 3, x 2, x 3).  A1 B1 + A2 B2 is then the
// product with the levels hi + lo.

// Eight codes of widths w <= 4 from the window x (code e at bits [e w, (e + 1) w)), two per
// lookup in the hi/lo pair table at byte offset tb.  o1, o2, o3 = 2w, 4w, 6w; w2 = 2w (the field
// extracts use bits 4:0 of each).
__device__ __forceinline__ void dec8_pairs(uint32_t x, uint32_t w2, uint32_t o1, uint32_t o2, uint32_t o3,
                                           uint32_t tb, const uint8_t* lds, u32x4& A1, u32x4& A2) {
  const uint32_t i0 = __builtin_amdgcn_ubfe(x, 0u, w2), i1 = __builtin_amdgcn_ubfe(x, o1, w2);
  const uint32_t i2 = __builtin_amdgcn_ubfe(x, o2, w2), i3 = __builtin_amdgcn_ubfe(x, o3, w2);
  const uint2 v0 = *reinterpret_cast<const uint2*>(lds + tb + 8 * i0);
  const uint2 v1 = *reinterpret_cast<const uint2*>(lds + tb + 8 * i1);
  const uint2 v2 = *reinterpret_cast<const uint2*>(lds + tb + 8 * i2);
  const uint2 v3 = *reinterpret_cast<const uint2*>(lds + tb + 8 * i3);
  A1 = u32x4{v0.x, v0.y, v1.x, v1.y};
  A2 = u32x4{v2.x, v2.y, v3.x, v3.y};
}

// The same for widths w <= 5 from the 64-bit window xh:xl (the fourth pair can cross bit 32).
__device__ __forceinline__ void dec8_pairs5(uint32_t xl, uint32_t xh, uint32_t w2, uint32_t o1, uint32_t o2,
                                            uint32_t o3, uint32_t tb, const uint8_t* lds, u32x4& A1, u32x4& A2) {
  const uint32_t x3 = __builtin_amdgcn_alignbit(xh, xl, o3);
  const uint32_t i0 = __builtin_amdgcn_ubfe(xl, 0u, w2), i1 = __builtin_amdgcn_ubfe(xl, o1, w2);
  const uint32_t i2 = __builtin_amdgcn_ubfe(xl, o2, w2), i3 = __builtin_amdgcn_ubfe(x3, 0u, w2);
  const uint2 v0 = *reinterpret_cast<const uint2*>(lds + tb + 8 * i0);
  const uint2 v1 = *reinterpret_cast<const uint2*>(lds + tb + 8 * i1);
  const uint2 v2 = *reinterpret_cast<const uint2*>(lds + tb + 8 * i2);
  const uint2 v3 = *reinterpret_cast<const uint2*>(lds + tb + 8 * i3);
  A1 = u32x4{v0.x, v0.y, v1.x, v1.y};
  A2 = u32x4{v2.x, v2.y, v3.x, v3.y};
}

// Eight codes of any width w (1..8) from the 64-bit window xh:xl, one per lookup in the hi | lo
// single table at byte offset tb.
__device__ __forceinline__ void dec8_singles(uint32_t xl, uint32_t xh, uint32_t w, uint32_t tb, const uint8_t* lds,
                                             u32x4& A1, u32x4& A2) {
  const uint64_t x = (uint64_t(xh) << 32) | xl;
  uint32_t v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t c = uint32_t(x >> (uint32_t(e) * w)) & ((1u << w) - 1u);   // e w + w <= 64
    v[e] = *reinterpret_cast<const uint32_t*>(lds + tb + 4 * c);
  }
  uint32_t o[8];
#pragma unroll
  for (int e2 = 0; e2 < 4; ++e2) {
    o[2 * e2] = __builtin_amdgcn_perm(v[2 * e2 + 1], v[2 * e2], 0x05040100u);       // hi of the pair
    o[2 * e2 + 1] = __builtin_amdgcn_perm(v[2 * e2 + 1], v[2 * e2], 0x07060302u);   // lo of the pair
  }
  A1 = u32x4{o[0], o[1], o[2], o[3]};
  A2 = u32x4{o[4], o[5], o[6], o[7]};
}

// Value codes decode to one fp16 term per level (the nearest fp16 of the fp32 centroid): the
// value sum is a convex combination of reconstructions, and the fp16 rounding of its levels
// moves the output by about 2^-12 relative, well inside the decode tolerance.  (The logits do
// need the hi + lo pair: a rounded key level shifts every logit, and sharp softmax rows amplify
// that.)  An MFMA operand then holds 8 consecutive codes' levels in k-slot order.

// Eight codes of width w <= 4 from the window x (pair k at bits [2 k w, 2 (k + 1) w)), two per
// b32 read of high-part pairs at byte offset tb, entries 1 << sh bytes apart.  o1..o3 = 2w, 4w,
// 6w; w2 = 2w.
__device__ __forceinline__ u32x4 vdec8_hpairs4(uint32_t x, uint32_t w2, uint32_t o1, uint32_t o2, uint32_t o3,
                                               uint32_t tb, uint32_t sh, const uint8_t* lds) {
  return u32x4{*reinterpret_cast<const uint32_t*>(lds + tb + (__builtin_amdgcn_ubfe(x, 0u, w2) << sh)),
               *reinterpret_cast<const uint32_t*>(lds + tb + (__builtin_amdgcn_ubfe(x, o1, w2) << sh)),
               *reinterpret_cast<const uint32_t*>(lds + tb + (__builtin_amdgcn_ubfe(x, o2, w2) << sh)),
               *reinterpret_cast<const uint32_t*>(lds + tb + (__builtin_amdgcn_ubfe(x, o3, w2) << sh))};
}
// Eight codes of width 5 from the 64-bit window xh:xl (the fourth pair can cross bit 32), two per
// b32 read of the high-part pairs of the hi/lo pair table at byte offset tb.
__device__ __forceinline__ u32x4 vdec8_hpairs(uint32_t xl, uint32_t xh, uint32_t w2, uint32_t o1, uint32_t o2,
                                              uint32_t o3, uint32_t tb, const uint8_t* lds) {
  const uint32_t x3 = __builtin_amdgcn_alignbit(xh, xl, o3);
  const uint32_t i0 = __builtin_amdgcn_ubfe(xl, 0u, w2), i1 = __builtin_amdgcn_ubfe(xl, o1, w2);
  const uint32_t i2 = __builtin_amdgcn_ubfe(xl, o2, w2), i3 = __builtin_amdgcn_ubfe(x3, 0u, w2);
  return u32x4{*reinterpret_cast<const uint32_t*>(lds + tb + 8 * i0), *reinterpret_cast<const uint32_t*>(lds + tb + 8 * i1),
               *reinterpret_cast<const uint32_t*>(lds + tb + 8 * i2), *reinterpret_cast<const uint32_t*>(lds + tb + 8 * i3)};
}
// Eight codes of any width w from the 64-bit window xh:xl, one per b32 read of the hi | lo single
// table at byte offset tb; the high parts (low halves) packed in pairs.
__device__ __forceinline__ u32x4 vdec8_hsingles(uint32_t xl, uint32_t xh, uint32_t w, uint32_t tb, const uint8_t* lds) {
  const uint64_t x = (uint64_t(xh) << 32) | xl;
  uint32_t v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t c = uint32_t(x >> (uint32_t(e) * w)) & ((1u << w) - 1u);   // e w + w <= 64
    v[e] = *reinterpret_cast<const uint32_t*>(lds + tb + 4 * c);
  }
  return u32x4{__builtin_amdgcn_perm(v[1], v[0], 0x05040100u), __builtin_amdgcn_perm(v[3], v[2], 0x05040100u),
               __builtin_amdgcn_perm(v[5], v[4], 0x05040100u), __builtin_amdgcn_perm(v[7], v[6], 0x05040100u)};
}

// Lanes l, l ^ 16, l ^ 32 and l ^ 48 combined by 16-lane row exchanges (VALU, no LDS traffic):
// the first swap pairs rows 0/1 and 2/3, the second the two halves of the wave.
__device__ __forceinline__ float rows_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows_sum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// B operand of the interleaved form from four values' fp16 halves packed as (x0 | x1 << 16,
// x2 | x3 << 16)
__device__ __forceinline__ f16x8 bdup(uint32_t x01, uint32_t x23) {
  return __builtin_bit_cast(f16x8, u32x4{x01, x01, x23, x23});
}

// k-step class: 0 = every segment at most 4 bits wide, 1 = at most 5, 2 = wider
__device__ __forceinline__ uint32_t seg_class(uint32_t w) { return w <= 4 ? 0u : (w == 5 ? 1u : 2u); }

template <int D, typename QT, bool STEP, bool ORDER>
__global__ __launch_bounds__(kStreamThreads) __attribute__((amdgpu_waves_per_eu(2)))
void k_decode_stream(DecodeArgs a, AppendArgs aa) {
  constexpr int MT = D / 16;                         // value M-tiles (16 coordinates each)
  constexpr int KS = tc_ksteps(D);                   // k-steps at most
  constexpr int SLOT = stream_slot_max(D);
  static_assert(KS <= kQRegSteps, "every k-step's operands in the prologue's B rows");
  __shared__ __align__(16) uint8_t s_tab[kSTabBytes];
  __shared__ __align__(16) uint4 s_kd[4 * kMaxKSteps];
  __shared__ float s_ml[2 * kStreamWaves * 8];
  __shared__ __align__(16) uint8_t s_pro[stream_pro_bytes(D)];
  __shared__ __align__(16) uint8_t s_ring0[kStreamWaves * SLOT];
  __shared__ __align__(16) uint8_t s_ring1[kStreamWaves * SLOT];
  // ORDER: a batch launch of several rounds, grid slots taken longest sequence first (a
  // separate instantiation, so that the one-round pass carries none of it)
  int s_slot = int(blockIdx.z);
  if constexpr (ORDER) s_slot = seq_longest_first(a.lengths, a.batch, reinterpret_cast<int*>(s_ml));
  const int s = s_slot;
  if constexpr (STEP) {
    if (blockIdx.x == 0) {          // decode step: workgroup 0 of every (sequence, KV head) appends
      if (aa.givens) step_append_role<false, true>(aa, a.step_flag, s, blockIdx.y, s_ring0);
      else step_append_role<false, false>(aa, a.step_flag, s, blockIdx.y, s_ring0);
      return;
    }
  }
  const int split = int(blockIdx.x) - (STEP ? 1 : 0), hk = blockIdx.y;
  const int group = keep_s(a.group), n_q = keep_s(a.n_q);
  const gptr<float> partial = keep_g(a.partial);
  const gptr<uint64_t> part_ml = keep_g(reinterpret_cast<uint64_t*>(a.part_ml));   // (max, sum) pairs
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, j = lane >> 4;
  // in a decode step the append role adds the new token beside this pass and the merge kernel
  // advances lengths[], so it still holds the old length here
  const int len0 = a.lengths[s];
  const int len = a.step && len0 + 1 <= a.capacity ? len0 + 1 : len0;
  const int n_ps = keep_s(a.n_split);
  // Work units: whole tiles round-robin over the waves of this (sequence, KV head) (wave
  // index vidx = split + n_ps * wave, W waves), and the remaining tiles cut into quarters, one
  // quarter per wave in the same order, so that any two waves' work differs by at most a quarter
  // of a tile.  Quarter q of a tile is its row block q: tokens 32 (q / 2) + 4 (q % 2) + 8 i + e,
  // i, e < 4.  Unit k < base of a wave is tile vidx + W k; unit k >= base is quarter
  // (vidx + (k - base) W) % 4 of tile base W + (vidx + (k - base) W) / 4.  (The quarters come
  // last: in a decode step the new token's unit is then a wave's last one, and its wait for the
  // append is over long before; taken first, that wait stalled the step.)
  const int tiles = (len + kTile - 1) / kTile;
  const int W = kStreamWaves * n_ps, vidx = split + n_ps * wave;
  const int base0 = tiles / W, rem = tiles - base0 * W;
  // a launch of several rounds of workgroups (a batch of many units) hands the remaining tiles
  // out whole, one more to waves vidx < rem: there the total work sets the time, and a quarter
  // costs more than a quarter of a tile and stages the whole tile
  const bool whole = keep_s(a.stream_whole_tiles) != 0;
  const int base = whole && vidx < rem ? base0 + 1 : base0;
  int nqu = !whole && 4 * rem > vidx ? (4 * rem - vidx + W - 1) / W : 0;
  if (nqu > 0) {              // a quarter of the last tile whose first token is past the length holds none
    const int u = vidx + (nqu - 1) * W;
    if (kTile * (base * W + u / 4) + 32 * ((u & 3) >> 1) + 4 * (u & 1) >= len) --nqu;
  }
  const int wcount = base + nqu;
  auto unit_tile = [&](int k) { return k < base ? vidx + W * k : base * W + (vidx + (k - base) * W) / 4; };
  auto unit_quarter = [&](int k) { return k < base ? -1 : (vidx + (k - base) * W) & 3; };
  // a decode step: the wave whose units include the new token's waits for the append role
  // before it requests that unit's tile
  int k_new = -1;
  if constexpr (STEP) {
    if (len == len0 + 1) {
      const int tn = len0 / kTile;
      int own, kk;
      if (whole || tn < base0 * W) {
        own = tn % W;
        kk = tn / W;
      } else {
        const int sl = len0 % kTile;                  // its slot: quarter 2 (sl / 32) + (sl / 4) % 2
        const int u = 4 * (tn - base0 * W) + 2 * (sl >> 5) + ((sl >> 2) & 1);
        own = u % W;
        kk = base0 + u / W;
      }
      if (own == vidx) k_new = kk;
    }
  }
  const int bv = keep_s(a.v_bits), chunks = keep_s(a.chunks);
  const StreamSlot geo = stream_slot(D, chunks, bv);
  const size_t reg = size_t(s) * a.n_kv + hk;
  const int64_t cap_tiles = a.capacity / kTile;
  const uint8_t* const kc = keep_s(a.k_codes + reg * cap_tiles * chunks * kTile * 16);
  const uint8_t* const knp = keep_s(reinterpret_cast<const uint8_t*>(a.k_norms + reg * cap_tiles * kMaxGroups * kTile));
  const uint8_t* const vnp = keep_s(reinterpret_cast<const uint8_t*>(a.v_norms + reg * cap_tiles * kTile));
  const uint8_t* const vc = keep_s(a.v_codes + reg * cap_tiles * D * 8 * bv);
  // K norm planes in use: one 128-byte plane per width group, 8 load lanes each (at least one
  // plane's lanes, so that every tile takes the same number of loads)
  const int kn_lanes = 8 * max(1, __builtin_amdgcn_readfirstlane(a.layouts[reg].n_groups));
  uint8_t* const slot0 = s_ring0 + wave * SLOT;
  uint8_t* const slot1 = s_ring1 + wave * SLOT;

  // ---- a tile into a slot: direct loads, 1 KiB per wave each, lane l's 16 bytes to slot +
  // base + 16 l.  Load i < chunks: K record unit u = 64 i + l (token u / chunks, chunk
  // u % chunks of the chunk-major HBM layout, so the slot holds token-major records); then the
  // K norm planes of the layout's groups; then the value units u (norms for u < 8, codes after),
  // lanes past the last unit off.
  const uint32_t inv_ch = (65536u + uint32_t(chunks) - 1u) / uint32_t(chunks > 0 ? chunks : 1);
  auto load_tile = [&](int k, uint8_t* slot) {     // the whole tile, also for a quarter unit
    const int tile = unit_tile(k);
    const uint8_t* kt = kc + size_t(tile) * chunks * kTile * 16;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i < chunks) {
        const uint32_t u = uint32_t(64 * i + lane), t = (u * inv_ch) >> 16, c = u - t * uint32_t(chunks);
        stage16(kt + (c * kTile + t) * 16, slot + 1024 * i);
      }
    }
    if (lane < kn_lanes) stage16(knp + size_t(tile) * (2 * kMaxGroups * kTile) + 16 * lane, slot + geo.kn_off);
#pragma unroll
    for (int i = 0; i < (D * 4 + 8 + 63) / 64; ++i) {   // up to 4 bits per value code
      if (i < geo.v_loads) {
        const int u = 64 * i + lane;
        if (u < geo.v_units) {
          const uint8_t* src = u < 8 ? vnp + size_t(tile) * (2 * kTile) + 16 * u
                                     : vc + size_t(tile) * D * 8 * bv + 16 * (u - 8);
          stage16(src, slot + geo.vn_off + 1024 * i);
        }
      }
    }
  };
  auto wait_append = [&]() {        // one wave: bounded wait for the append role, then acquire
    if (lane == 0) {
      const int32_t* f = a.step_flag + (size_t(s) * a.n_kv + hk);
      int i = 0;
      for (; i < a.step_spin; ++i) {
        if (__hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == len0 + 1) break;
        __builtin_amdgcn_s_sleep(2);
      }
      if (i == a.step_spin && aa.status) atomicOr(aa.status, 2);   // gave up: reported
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  };

  // ---- workgroup set-up and query prologue (the matrix-core pass's helpers, on the first 256
  // threads).  Global reads in two rounds: what does not depend on the layout descriptor
  // (descriptor, tables, query), then the rotation rows; the wave's first two tiles are
  // requested between the two.
  constexpr int NP = QShape<D>::NP, QI = QShape<D>::QI;
  constexpr int PW = (kPairWords + kStreamThreads - 1) / kStreamThreads;
  constexpr int SW = (kSingleHalves + kStreamThreads - 1) / kStreamThreads;
  static_assert(BGTQ_LAYOUT_BYTES == 256 * 16, "one 16-byte piece of the layout per thread of the first 256");
  HeadLayout* const Ls = reinterpret_cast<HeadLayout*>(s_pro);
  float* const qc = reinterpret_cast<float*>(s_pro + BGTQ_LAYOUT_BYTES);                 // q' [coordinate][8 heads]
  uint4* const qhi = reinterpret_cast<uint4*>(s_pro + BGTQ_LAYOUT_BYTES + 32 * D);       // [k-step][lane]
  uint4* const qlo = qhi + 64 * kQRegSteps;                                            // [k-step][lane]
  const HeadLayout* L = a.layouts + reg;
  {
    uint4 lw = uint4{0u, 0u, 0u, 0u};
    if (tid < 256) lw = reinterpret_cast<const uint4*>(L)[tid];
    uint2 pt[PW];
    uint32_t st[SW];
#pragma unroll
    for (int i = 0; i < PW; ++i)
      if (tid + kStreamThreads * i < kPairWords) pt[i] = c_pair_hl[tid + kStreamThreads * i];
#pragma unroll
    for (int i = 0; i < SW; ++i)
      if (tid + kStreamThreads * i < kSingleHalves) st[i] = c_single_hl[tid + kStreamThreads * i];
    float x0[QI], x1[QI];
    double fr = 0.0;
    if (tid < 256) {
      q_load<D, QT>(a, s, hk, tid, x0, x1);
      fr = a.rope_theta > 0.0 ? a.inv_freq[tid % NP] : 0.0;
    }
    if (tid < 256) reinterpret_cast<uint4*>(Ls)[tid] = lw;
#pragma unroll
    for (int i = 0; i < PW; ++i)
      if (tid + kStreamThreads * i < kPairWords) reinterpret_cast<uint2*>(s_tab + kSTabPair)[tid + kStreamThreads * i] = pt[i];
    if (tid < kVPairWords) reinterpret_cast<uint32_t*>(s_tab + kSTabV)[tid] = pt[0].x;
#pragma unroll
    for (int i = 0; i < SW; ++i)
      if (tid + kStreamThreads * i < kSingleHalves) reinterpret_cast<uint32_t*>(s_tab + kSTabSingle)[tid + kStreamThreads * i] = st[i];
    if (tid < 256) {
      qops_zero(qhi, qlo, qlo + 64 * kQRegSteps, KS, tid);
      q_rope<D>(a, a.q_pos ? a.q_pos[s] : int64_t(len) - 1, fr, tid, x0, x1, qc);
    }
  }
  if (wcount > 0 && k_new != 0) load_tile(0, slot0);
  if (wcount > 1 && k_new != 1) load_tile(1, slot1);
  lds_barrier();
  // dense rotations: q''_p = (softmax_scale log2(e) / sqrt(m)) sum_c R_m[p - first][c] q'[perm[first + c]]
  // for storage position p = tid / 4; the four threads of p take a quarter of the row each
  // (float2 pairs of coordinates), their rows requested first (the addresses take dependent
  // reads of the layout), before the k-step descriptors are built
  const bool giv = a.givens != nullptr;
  constexpr int RQ = D / 8;                          // float2 of a row quarter at most (m <= D)
  const int rp = tid >> 2, rk = tid & 3, d_eff = Ls->d_eff;
  float2 rq[RQ];
  int rm = 2, rfirst = 0, rb0 = 0, rn = 0;
  if (!giv && rp < d_eff) {
    const int g = Ls->group[rp];
    rm = Ls->g_m[g];
    rfirst = Ls->g_first[g];
    const int per = (rm / 2 + 3) / 4;
    rb0 = rk * per;
    rn = min(per, rm / 2 - rb0);
    const float2* R2 = reinterpret_cast<const float2*>(a.rot_bank + bank_offset(rm) + size_t(rp - rfirst) * rm) + rb0;
#pragma unroll
    for (int i = 0; i < RQ; ++i)
      if (i < rn) rq[i] = R2[i];
  }
  const int nks = Ls->n_ksteps;
  const uint32_t wmask = wide_ksteps(Ls, nks, lane);
  const int nn = nks - __popc(wmask);               // narrow k-steps
  // per k-step (kernel order: narrow ones first) and lane group j: x = byte offset of the
  // window's first record dword, y = shift | 2w << 8 | 4w << 16 | 6w << 24, z = byte offset of
  // the width's pair table (w <= 5), w = byte offset of its single table | w << 16 | class << 20 |
  // first group << 24 | second group << 28 (class 0: every segment of the k-step at most 4 bits
  // wide, 1: at most 5, 2: wider, decoded one code per lookup; the groups name the K norm planes
  // of output columns 0-7 and 8-15)
  for (int i = tid; i < 4 * nks; i += kStreamThreads) {
    const int ks = i >> 2;
    const uint32_t seg = Ls->seg[i];
    const uint32_t o = seg & 0xffffu, w = (seg >> 16) & 15u;
    uint32_t wmax = 0;
#pragma unroll
    for (int sl = 0; sl < 4; ++sl) wmax = max(wmax, (Ls->seg[4 * ks + sl] >> 16) & 15u);
    const uint32_t kg = Ls->kgroups[ks];
    const uint32_t tbp = w <= 5 ? uint32_t(kSTabPair + 8 * pair_base(int(w))) : 0u;
    const uint32_t tbs = uint32_t(kSTabSingle + 4 * single_base(int(w)));
    s_kd[4 * kperm_of(wmask, nn, ks) + (i & 3)] =
        uint4{4u * (o >> 5), (o & 31u) | (2u * w) << 8 | (4u * w) << 16 | (6u * w) << 24, tbp,
              tbs | w << 16 | seg_class(wmax) << 20 | (kg & 7u) << 24 | ((kg >> 8) & 7u) << 28};
  }
  if (giv) {
    qops_givens_rotate(a, Ls, qc, tid, 256);     // every thread: it holds the barriers
    if (tid < 256) qops_scatter_rotated<true>(a, Ls, qc, wmask, nn, tid, qhi, qlo, qlo + 64 * kQRegSteps);
  } else if (rp < d_eff) {
    float acc[8];
#pragma unroll
    for (int h = 0; h < 8; ++h) acc[h] = 0.0f;
    const uint8_t* pm = Ls->perm + rfirst + 2 * rb0;
#pragma unroll
    for (int i = 0; i < RQ; ++i) {
      if (i < rn) {
        const float4* xa = reinterpret_cast<const float4*>(qc + 8 * pm[2 * i]);
        const float4* xb = reinterpret_cast<const float4*>(qc + 8 * pm[2 * i + 1]);
        const float4 a0 = xa[0], a1 = xa[1], c0 = xb[0], c1 = xb[1];
        const float r0 = rq[i].x, r1 = rq[i].y;
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
    // the quarters' sums (pairwise within the quad, so the four threads agree), then heads 2 rk, 2 rk + 1 of p
    // into the B operand slots of p's k-step: fp16 high part and remainder
#pragma unroll
    for (int h = 0; h < 8; ++h) {
      acc[h] += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, acc[h]), 0xB1, 0xf, 0xf, false));   // lane ^ 1
      acc[h] += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, acc[h]), 0x4E, 0xf, 0xf, false));   // lane ^ 2
    }
    const float f = a.scale * kLog2e / sqrtf(float(rm));
    const int kx = Ls->kpos[rp], ks0 = kx >> 5, jj = (kx >> 3) & 3, e = kx & 7, ks = kperm_of(wmask, nn, ks0);
    const int lb = 16 * jj + 8 * int((Ls->seg[4 * ks0 + jj] >> 28) & 1u);
    uint16_t* q16 = reinterpret_cast<uint16_t*>((e < 4 ? qhi : qlo) + 64 * ks);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int h = 2 * rk + hh;
      if (h < group) {
        const float v = (rk == 0 ? acc[hh] : rk == 1 ? acc[2 + hh] : rk == 2 ? acc[4 + hh] : acc[6 + hh]) * f;
        const uint16_t hi = f32_to_f16_bits(v);
        q16[(lb + h) * 8 + (e & 3)] = hi;
        q16[(lb + h) * 8 + 4 + (e & 3)] = f32_to_f16_bits(v - f16_bits_to_f32(hi));
      }
    }
  }
  // value quads of widths 1 and 2 (entry c0 | c1 << w | c2 << 2w | c3 << 3w: the fp16 levels of
  // the four codes), built from the single table's high parts
  if (tid < kVQuadWords) {
    const int w = tid < 16 ? 1 : 2, i = tid < 16 ? tid : tid - 16, mk = (1 << w) - 1;
    const uint32_t* sg = reinterpret_cast<const uint32_t*>(s_tab + kSTabSingle) + single_base(w);
    const uint32_t l0 = sg[i & mk] & 0xffffu, l1 = sg[(i >> w) & mk] & 0xffffu;
    const uint32_t l2 = sg[(i >> (2 * w)) & mk] & 0xffffu, l3 = sg[(i >> (3 * w)) & mk] & 0xffffu;
    reinterpret_cast<uint2*>(s_tab + kSTabVQ)[tid] = uint2{l0 | l1 << 16, l2 | l3 << 16};
  }
  lds_barrier();

  // ---- per-lane constants
  const uint32_t rec = uint32_t(16 * chunks);
  const uint32_t krow = uint32_t(8 * (n >> 2) + (n & 3)) * rec;      // token 8 (n / 4) + n % 4, row block 0
  const uint32_t kr1 = 4u * rec, kr2 = 32u * rec, kr3 = 36u * rec;   // row blocks 1..3: + 4, 32, 36 tokens
  const uint32_t nsh = n < 8 ? 24u : 28u;                            // the lane's norm group field of d.w
  const uint32_t knb = uint32_t(geo.kn_off + 2 * 8 * j);             // tokens 8 j .. 8 j + 7 of a norm plane
  // value windows: coordinate 16 mt + n, tokens 32 b + 8 j .. + 7: bits (32 b + 8 j) b_v of the
  // coordinate's segment of 8 b_v bytes
  const uint32_t vwin = uint32_t(geo.vc_off + n * 8 * bv + 4 * ((8 * j * bv) >> 5));
  const uint32_t vctl = uint32_t((8 * j * bv) & 31) | (2u * bv) << 8 | (4u * bv) << 16 | (6u * bv) << 24;
  const uint32_t vmt = uint32_t(16 * 8 * bv);                        // bytes between M-tiles
  // value pair lookups of widths <= 3 read the compact high-part table (4-byte entries, so that
  // neighbouring entries fall on neighbouring banks); width 4 the high halves of the hi/lo pairs
  const uint32_t vtb = bv <= 3 ? uint32_t(kSTabV + 4 * pair_base(bv))
                               : bv <= 5 ? uint32_t(kSTabPair + 8 * pair_base(bv)) : uint32_t(kSTabSingle + 4 * single_base(bv));
  const uint32_t vsh = bv <= 3 ? 2u : 3u;
  // value decode, from the high parts of the key tables: 0 = widths <= 4, pairs from a 32-bit
  // window; 1 = width 5, pairs from a 64-bit window; 2 = wider, singles
  const uint32_t vmode = bv <= 4 ? 0u : (bv == 5 ? 1u : 2u);
  // widths 1 and 2 read four codes per lookup from the quad table
  const bool vquad = bv <= 2;
  const uint32_t vqb = uint32_t(kSTabVQ + 8 * (bv == 1 ? 0 : 16));

  f32x4 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_part = 0.0f;
  const bool real_col = n < group;
  const gptr<float> logits = keep_g(a.logits);
  const int64_t capacity = keep_s(a.capacity);

  auto ld32 = [](const uint8_t* p) { return *reinterpret_cast<const uint32_t*>(p); };

  // ---- one work unit from its slot: logits (the unit's row blocks per k-step), online softmax,
  // P V.  NRB = 4: a whole tile (row blocks 0..3, value blocks 0, 1); NRB = 1: quarter rb0 of a
  // tile (row block rb0, half rb0 % 2 of value block rb0 / 2).  Within a k-step the row blocks'
  // reads are issued together (the k-step's class is uniform, so the decode form is chosen once
  // per k-step), and the next k-step's descriptor and B operands are requested one k-step ahead.
  auto process_unit = [&](auto nrb_c, int tile, int rb0, const uint8_t* slot) {
    constexpr int NRB = decltype(nrb_c)::value;
    static_assert(NRB == 4 || NRB == 1, "whole tiles and quarters");
    const int valid = len - tile * kTile < kTile ? len - tile * kTile : kTile;   // the tile's tokens
    const int tk0 = 32 * (rb0 >> 1) + 4 * (rb0 & 1);   // row 0 of the unit's first row block
    const int tb0 = 32 * (rb0 >> 1);                   // the unit's first 32-token value block
    f32x4 S[NRB];
#pragma unroll
    for (int q = 0; q < NRB; ++q) S[q] = f32x4{0.f, 0.f, 0.f, 0.f};
    const uint8_t* kw = slot + krow + uint32_t(tk0) * rec;
    const uint32_t ro[4] = {0u, kr1, kr2, kr3};      // row block q of the unit: + ro[q]
    // one k-step: descriptor d, B operands qa (k slots 0..3) and qb (4..7)
    auto kstep = [&](const uint4& d, const uint4& qa, const uint4& qb) {
      const uint32_t cls = (__builtin_amdgcn_readfirstlane(d.w) >> 20) & 3u;   // the same for every lane group
      const uint8_t* np = slot + knb + 128u * __builtin_amdgcn_ubfe(d.w, nsh, 3u) + 2u * uint32_t(tb0);
      uint4 nq[(NRB + 1) / 2];                           // K norms of row blocks 2 i, 2 i + 1 (of the unit's block)
#pragma unroll
      for (int i = 0; i < (NRB + 1) / 2; ++i) nq[i] = *reinterpret_cast<const uint4*>(np + 64 * i);
      const uint8_t* kb = kw + d.x;
      const uint32_t w2 = d.y >> 8, o2 = d.y >> 16, o3 = d.y >> 24;   // the field extracts use bits 4:0
      u32x4 A1[NRB], A2[NRB];
      if (cls == 0u) {
        uint32_t wa[NRB], wb[NRB];
#pragma unroll
        for (int q = 0; q < NRB; ++q) {
          wa[q] = ld32(kb + ro[q]);
          wb[q] = ld32(kb + ro[q] + 4);
        }
#pragma unroll
        for (int q = 0; q < NRB; ++q) dec8_pairs(win32(wa[q], wb[q], d.y), w2, w2, o2, o3, d.z, s_tab, A1[q], A2[q]);
      } else {
        uint32_t wa[NRB], wb[NRB], wc[NRB];
#pragma unroll
        for (int q = 0; q < NRB; ++q) {
          wa[q] = ld32(kb + ro[q]);
          wb[q] = ld32(kb + ro[q] + 4);
          wc[q] = ld32(kb + ro[q] + 8);
        }
        if (cls == 1u) {
#pragma unroll
          for (int q = 0; q < NRB; ++q)
            dec8_pairs5(win32(wa[q], wb[q], d.y), win32(wb[q], wc[q], d.y), w2, w2, o2, o3, d.z, s_tab, A1[q], A2[q]);
        } else {
#pragma unroll
          for (int q = 0; q < NRB; ++q)
            dec8_singles(win32(wa[q], wb[q], d.y), win32(wb[q], wc[q], d.y), (d.w >> 16) & 15u, d.w & 0xffffu, s_tab,
                         A1[q], A2[q]);
        }
      }
      const f16x8 B1h = bdup(qa.x, qa.y), B1l = bdup(qa.z, qa.w), B2h = bdup(qb.x, qb.y), B2l = bdup(qb.z, qb.w);
#pragma unroll
      for (int q = 0; q < NRB; ++q) {
        const f16x8 a1 = __builtin_bit_cast(f16x8, A1[q]), a2 = __builtin_bit_cast(f16x8, A2[q]);
        f32x4 T = {0.f, 0.f, 0.f, 0.f};
        T = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, B1h, T, 0, 0, 0);
        T = __builtin_amdgcn_mfma_f32_16x16x32_f16(a2, B2h, T, 0, 0, 0);
        T = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, B1l, T, 0, 0, 0);
        T = __builtin_amdgcn_mfma_f32_16x16x32_f16(a2, B2l, T, 0, 0, 0);
        const uint4& nqq = nq[q >> 1];
        const bool odd = NRB == 1 ? (rb0 & 1) != 0 : (q & 1) != 0;   // the second row block of its pair
        const f16x4 nv = __builtin_bit_cast(f16x4, odd ? uint2{nqq.z, nqq.w} : uint2{nqq.x, nqq.y});
#pragma unroll
        for (int r = 0; r < 4; ++r) S[q][r] = fmaf(T[r], float(nv[r]), S[q][r]);
      }
    };
    // k-steps in pairs, each pair's operands requested one k-step ahead into two register sets
    uint4 d0 = s_kd[j], qa0 = qhi[lane], qb0 = qlo[lane];
    uint4 d1 = d0, qa1 = qa0, qb1 = qb0;
    for (int ks = 0; ks < nks; ks += 2) {
      if (ks + 1 < nks) {
        d1 = s_kd[4 * (ks + 1) + j];
        qa1 = qhi[64 * (ks + 1) + lane];
        qb1 = qlo[64 * (ks + 1) + lane];
      }
      kstep(d0, qa0, qb0);
      if (ks + 1 < nks) {
        if (ks + 2 < nks) {
          d0 = s_kd[4 * (ks + 2) + j];
          qa0 = qhi[64 * (ks + 2) + lane];
          qb0 = qlo[64 * (ks + 2) + lane];
        }
        kstep(d1, qa1, qb1);
      }
    }

    // online softmax (base 2).  Head c = column c + column c + 8 (row rotation by 8, so both
    // lanes hold the head's logit); lane (c, j) holds tokens 32 (rb / 2) + 8 j + 4 (rb % 2) + r
    // of the tile's row block rb = rb0 + q (the unit's q-th).
    float v[NRB][4];
#pragma unroll
    for (int q = 0; q < NRB; ++q) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float sr = S[q][r];
        const float other = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, sr), 0x128, 0xf, 0xf, false));
        v[q][r] = sr + other;
      }
    }
    if (valid < tb0 + (NRB == 4 ? 64 : 32)) {     // the unit passes the sequence's end (its last tile only)
#pragma unroll
      for (int q = 0; q < NRB; ++q)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (32 * ((rb0 + q) >> 1) + 8 * j + 4 * ((rb0 + q) & 1) + r >= valid) v[q][r] = -INFINITY;
    }
    float lm = -INFINITY;
#pragma unroll
    for (int q = 0; q < NRB; ++q)
#pragma unroll
      for (int r = 0; r < 4; ++r) lm = fmaxf(lm, v[q][r]);
    if (logits && real_col) {
      const gptr<float> lg = logits + (int64_t(s) * n_q + hk * group + n) * capacity + int64_t(tile) * kTile + 8 * j;
#pragma unroll
      for (int q = 0; q < NRB; ++q)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 32 * ((rb0 + q) >> 1) + 4 * ((rb0 + q) & 1) + r;
          if (t + 8 * j < valid) lg[t] = v[q][r] * kLn2;
        }
    }
    lm = rows_max(lm);
    const float m_new = fmaxf(m_run, lm);            // finite: every unit has a valid token
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    float psum = 0.0f;
#pragma unroll
    for (int q = 0; q < NRB; ++q)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        v[q][r] = __builtin_amdgcn_exp2f(v[q][r] - m_new);
        psum += v[q][r];
      }
    l_part = l_part * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] *= alpha;   // unconditional: a skip branch cost register copies
    // P V: value block b (tokens 32 b ..), k slot 8 j + e = token 32 b + 8 j + e: row block
    // 2 b (e < 4) and 2 b + 1 (e >= 4); P n_v in fp16, in the interleaved B form (a quarter's
    // other row block enters as zeros).  The M-tiles' windows and lookups are issued together.
#pragma unroll
    for (int bl = 0; bl < (NRB == 4 ? 2 : 1); ++bl) {
      const int b = NRB == 4 ? bl : (rb0 >> 1);
      if (32 * b < valid) {
        const f16x8 vn = *reinterpret_cast<const f16x8*>(slot + geo.vn_off + 2 * (32 * b + 8 * j));
        f16x8 P;
#pragma unroll
        for (int e = 0; e < 8; ++e) {    // the product (p, n_v >= 0), one mixed-precision op
          if constexpr (NRB == 4) {
            P[e] = (_Float16)fmaf(v[2 * bl + (e >> 2)][e & 3], float(vn[e]), 0.0f);
          } else {
            P[e] = (e >> 2) == (rb0 & 1) ? (_Float16)fmaf(v[0][e & 3], float(vn[e]), 0.0f) : (_Float16)0.0f;
          }
        }
        if (valid < kTile) {       // slots past the length: p is 0, their value norm may be any bits
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (32 * b + 8 * j + e >= valid) P[e] = (_Float16)0.0f;
        }
        const uint8_t* vb = slot + vwin + uint32_t(4 * b * bv);
        u32x4 VA[MT];
        if (vmode == 0u) {             // b_v <= 4: one 32-bit window per 8 codes
          uint32_t wa[MT], wb[MT];
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            wa[mt] = ld32(vb + mt * vmt);
            wb[mt] = ld32(vb + mt * vmt + 4);
          }
          const uint32_t w2 = vctl >> 8, o2 = vctl >> 16, o3 = vctl >> 24;   // 2 b_v, 4 b_v, 6 b_v (bits 4:0)
          if (vquad) {                 // quads: codes 0..3 at bit 0, codes 4..7 at bit 4 b_v
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
              const uint32_t x = win32(wa[mt], wb[mt], vctl);
              if constexpr (NRB == 1) {   // a quarter: its row block's four codes, repeated in the other half
                const uint2 c = *reinterpret_cast<const uint2*>(s_tab + vqb + 8 * __builtin_amdgcn_ubfe(x, (rb0 & 1) ? o2 : 0u, o2));
                VA[mt] = u32x4{c.x, c.y, c.x, c.y};
              } else {
                const uint2 c0 = *reinterpret_cast<const uint2*>(s_tab + vqb + 8 * __builtin_amdgcn_ubfe(x, 0u, o2));
                const uint2 c1 = *reinterpret_cast<const uint2*>(s_tab + vqb + 8 * __builtin_amdgcn_ubfe(x, o2, o2));
                VA[mt] = u32x4{c0.x, c0.y, c1.x, c1.y};
              }
            }
          } else if constexpr (NRB == 1) {    // a quarter: its row block's four codes, repeated in the other half
            const bool hi = (rb0 & 1) != 0;
            const uint32_t oa = hi ? o2 : 0u, ob = hi ? o3 : w2;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
              const uint32_t x = win32(wa[mt], wb[mt], vctl);
              const uint32_t c0 = *reinterpret_cast<const uint32_t*>(s_tab + vtb + (__builtin_amdgcn_ubfe(x, oa, w2) << vsh));
              const uint32_t c1 = *reinterpret_cast<const uint32_t*>(s_tab + vtb + (__builtin_amdgcn_ubfe(x, ob, w2) << vsh));
              VA[mt] = u32x4{c0, c1, c0, c1};
            }
          } else {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
              VA[mt] = vdec8_hpairs4(win32(wa[mt], wb[mt], vctl), w2, w2, o2, o3, vtb, vsh, s_tab);
          }
        } else {                       // wider: high parts from the LDS tables
          uint32_t wa[MT], wb[MT], wc[MT];
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            wa[mt] = ld32(vb + mt * vmt);
            wb[mt] = ld32(vb + mt * vmt + 4);
            wc[mt] = ld32(vb + mt * vmt + 8);
          }
          if (vmode == 1u) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
              VA[mt] = vdec8_hpairs(win32(wa[mt], wb[mt], vctl), win32(wb[mt], wc[mt], vctl), vctl >> 8, vctl >> 8,
                                    vctl >> 16, vctl >> 24, vtb, s_tab);
          } else {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
              VA[mt] = vdec8_hsingles(win32(wa[mt], wb[mt], vctl), win32(wb[mt], wc[mt], vctl), uint32_t(bv), vtb, s_tab);
          }
        }
        // P n_v is zero in the k slots of a quarter's other row block and past the length, so
        // whatever finite levels A holds there add nothing
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, VA[mt]), P, acc[mt], 0, 0, 0);
      }
    }
  };

  // ---- the wave's units, two slots: unit k in slot k % 2.  Unit m's tile is requested in the
  // prologue (m < 2), once the wave has read unit m - 2 out of the same slot, or, for the new
  // token's unit of a decode step, after the wait for the append role.  The waits for a slot's
  // loads are explicit: with unit k + 1 requested before unit k is processed, unit k is complete
  // once at most `ni` (unit k + 1's load count) vector memory operations are outstanding.
  const int ni = chunks + 1 + geo.v_loads;
  auto wait_tile = [&](int k) {
    const bool next = k + 1 < wcount && !(STEP && (k + 1 == k_new || k == k_new));
    if (!next) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    } else {
      switch (ni) {     // the count is an immediate of the instruction
        case 2: asm volatile("s_waitcnt vmcnt(2)" ::: "memory"); break;
        case 3: asm volatile("s_waitcnt vmcnt(3)" ::: "memory"); break;
        case 4: asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); break;
        case 5: asm volatile("s_waitcnt vmcnt(5)" ::: "memory"); break;
        case 6: asm volatile("s_waitcnt vmcnt(6)" ::: "memory"); break;
        case 7: asm volatile("s_waitcnt vmcnt(7)" ::: "memory"); break;
        case 8: asm volatile("s_waitcnt vmcnt(8)" ::: "memory"); break;
        case 9: asm volatile("s_waitcnt vmcnt(9)" ::: "memory"); break;
        case 10: asm volatile("s_waitcnt vmcnt(10)" ::: "memory"); break;
        case 11: asm volatile("s_waitcnt vmcnt(11)" ::: "memory"); break;
        case 12: asm volatile("s_waitcnt vmcnt(12)" ::: "memory"); break;
        case 13: asm volatile("s_waitcnt vmcnt(13)" ::: "memory"); break;
        case 14: asm volatile("s_waitcnt vmcnt(14)" ::: "memory"); break;
        default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
      }
    }
  };
  for (int k = 0; k < wcount; ++k) {
    uint8_t* const slot = (k & 1) ? slot1 : slot0;
    if (STEP && k == k_new) {      // the new token's tile: requested after the append role's release
      wait_append();
      load_tile(k, slot);
    }
    wait_tile(k);
    const int tile = unit_tile(k), qr = unit_quarter(k);
    if (qr < 0) process_unit(std::integral_constant<int, 4>{}, tile, 0, slot);
    else process_unit(std::integral_constant<int, 1>{}, tile, qr, slot);
    if (k + 2 < wcount && !(STEP && k + 2 == k_new)) {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");     // every read of the slot done
      load_tile(k + 2, slot);
    }
  }

  // ---- merge of the 8 waves: running maxima and sums through LDS, then each wave's
  // accumulator scaled to the common maximum, summed in wave order.  Lane (c, j) holds head
  // c % 8, coordinates 16 mt + 4 j + r.  The lane indices are taken afresh (opaque copies).
  // The split's partial result is stored at device scope (written through the L2), which leaves
  // the end of the pass less to write back before the merge kernel reads it (≈1% per call).
  int le = lane;
  asm volatile("" : "+v"(le));
  const int ne = le & 15, je = le >> 4;
  float l = l_part;
  l = rows_sum(l);
  float* mws = s_ml;                               // [8 waves][8 heads]
  float* lws = s_ml + 8 * kStreamWaves;
  if (je == 0 && ne < 8) {
    mws[8 * wave + ne] = m_run;
    lws[8 * wave + ne] = l;
  }
  __syncthreads();             // every wave is past its tiles: ring 0 is free for the merge
  float mmax = -INFINITY;
#pragma unroll
  for (int w = 0; w < kStreamWaves; ++w) mmax = fmaxf(mmax, mws[8 * w + (ne & 7)]);
  const float sc = m_run == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run - mmax);
  // [8 waves][8 heads][D + 16]: the padding puts the 8 heads' rows 16 banks apart, so that a
  // wave's 16-byte writes meet at most two to a bank (rows D floats apart all fell on the same
  // banks, and the writes cost more than the rest of the merge)
  constexpr int RS = D + 16;
  float* accw = reinterpret_cast<float*>(s_ring0);
  static_assert(kStreamWaves * 8 * RS * 4 <= kStreamWaves * SLOT, "the merge fits ring 0");
  if (ne < 8) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      *reinterpret_cast<float4*>(accw + (8 * wave + ne) * RS + 16 * mt + 4 * je) =
          float4{acc[mt][0] * sc, acc[mt][1] * sc, acc[mt][2] * sc, acc[mt][3] * sc};
  }
  __syncthreads();
  for (int i = tid; i < group * D; i += kStreamThreads) {
    const int h = i / D, r = i - h * D;
    float x = 0.0f;
#pragma unroll
    for (int w = 0; w < kStreamWaves; ++w) x += accw[(8 * w + h) * RS + r];
    const int64_t row = (int64_t(s) * n_q + hk * group + h) * n_ps + split;
    __hip_atomic_store(&partial[row * D + r], x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);   // written through: read by the merge kernel
  }
  if (tid < group) {
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < kStreamWaves; ++w) mx = fmaxf(mx, mws[8 * w + tid]);
    float lsum = 0.0f;
#pragma unroll
    for (int w = 0; w < kStreamWaves; ++w) {
      const float mw = mws[8 * w + tid];
      lsum += mw == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mw - mx) * lws[8 * w + tid];
    }
    const int64_t row = (int64_t(s) * n_q + hk * group + tid) * n_ps + split;
    __hip_atomic_store(&part_ml[row], uint64_t(__float_as_uint(mx)) | uint64_t(__float_as_uint(lsum)) << 32,
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}
