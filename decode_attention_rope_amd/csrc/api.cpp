// C ABI of the Block-GTQ packed-cache decode path: argument checks, sizes, launches.
// Declared and documented in include/bgtq.h.

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>

#include "bgtq_internal.h"

using namespace bgtq;

namespace {

thread_local std::string g_last_error;
std::mutex g_init_mutex;
bool g_device_ready[64] = {};
void* g_scratch[64] = {};     // device address of each GPU's allocation-free scratch

// process-wide options (bgtq_set_option); defaults from the environment, read once
std::atomic<int> g_decode_kernel{0};   // 0 automatic, 1 vector ALU, 2 tiled matrix-core pass
std::atomic<int> g_step_spin{1 << 22};
std::once_flag g_env_once;

bgtq_status fail(bgtq_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
bgtq_status fail(bgtq_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

bgtq_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return BGTQ_OK;
  return fail(BGTQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// The library's initialisation, once per device (the current one): the codebook tables go to
// constant memory and the device address of the allocation-free scratch is looked up.  The
// first initialisation in the process also takes the options' defaults from the environment;
// no other place reads it.
bgtq_status ensure_init() {
  std::call_once(g_env_once, [] {
    if (const char* k = std::getenv("BGTQ_DECODE_KERNEL"))
      g_decode_kernel = std::strcmp(k, "valu") == 0 ? 1 : std::strcmp(k, "tiled") == 0 ? 2 : 0;
    if (const char* sl = std::getenv("BGTQ_STEP_SPIN_LIMIT")) g_step_spin = std::atoi(sl) > 0 ? std::atoi(sl) : 0;
  });
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= 64) return fail(BGTQ_ERR_UNSUPPORTED, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_init_mutex);
  if (g_device_ready[dev]) return BGTQ_OK;
  e = upload_tables(host_tables());
  if (e != hipSuccess) return hip_status(e, "upload codebook tables");
  e = scratch_address(&g_scratch[dev]);
  if (e != hipSuccess) return hip_status(e, "scratch symbol address");
  g_device_ready[dev] = true;
  return BGTQ_OK;
}

bool head_dim_ok(int d) { return d >= 2 && d <= BGTQ_MAX_HEAD_DIM && d % 2 == 0; }

bgtq_status check_cache(const bgtq_cache* c, bool need_layout) {
  if (!c) return fail(BGTQ_ERR_INVALID_ARG, "cache is NULL");
  if (c->batch < 1 || c->n_kv_heads < 1) return fail(BGTQ_ERR_INVALID_ARG, "batch and n_kv_heads must be >= 1");
  if (!head_dim_ok(c->head_dim)) return fail(BGTQ_ERR_INVALID_ARG, "head_dim %d must be even, 2..256", c->head_dim);
  if (c->v_bits < 1 || c->v_bits > BGTQ_MAX_BITS) return fail(BGTQ_ERR_INVALID_ARG, "v_bits must be 1..8");
  if (c->k_width_sum < 0 || c->k_width_sum > BGTQ_MAX_BITS * (c->head_dim / 2))
    return fail(BGTQ_ERR_BUDGET, "k_width_sum %d outside [0, 8 * head_dim/2]", c->k_width_sum);
  if (c->capacity < kTile || c->capacity % kTile)
    return fail(BGTQ_ERR_INVALID_ARG, "capacity must be a positive multiple of 64");
  if (c->capacity > (int64_t(1) << 31) - 64) return fail(BGTQ_ERR_INVALID_ARG, "capacity too large");
  if (c->pairing != BGTQ_PAIR_HALF && c->pairing != BGTQ_PAIR_INTERLEAVED)
    return fail(BGTQ_ERR_INVALID_ARG, "bad pairing");
  if (!c->k_codes && c->k_width_sum > 0) return fail(BGTQ_ERR_INVALID_ARG, "k_codes is NULL");
  if (!c->k_norms || !c->v_codes || !c->v_norms || !c->lengths)
    return fail(BGTQ_ERR_INVALID_ARG, "cache arrays must not be NULL");
  if (need_layout && !c->layouts) return fail(BGTQ_ERR_INVALID_ARG, "layouts is NULL");
  if (c->window < 0 || c->window > BGTQ_MAX_WINDOW)
    return fail(BGTQ_ERR_INVALID_ARG, "window %d outside [0, %d]", c->window, BGTQ_MAX_WINDOW);
  if (c->window > 0 && !c->k_window) return fail(BGTQ_ERR_INVALID_ARG, "k_window is NULL");
  return BGTQ_OK;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

bgtq_status check_quantizer(const bgtq_quantizer* qz) {
  if (!qz) return fail(BGTQ_ERR_INVALID_ARG, "quantizer is NULL");
  if (qz->rotation == BGTQ_ROT_DENSE) {
    if (!qz->rot_bank || !qz->rot_v || !qz->rot_bank_t || !qz->rot_v_t)
      return fail(BGTQ_ERR_INVALID_ARG, "quantizer rotations are NULL");
  } else if (qz->rotation == BGTQ_ROT_GIVENS) {
    if (!qz->givens) return fail(BGTQ_ERR_INVALID_ARG, "quantizer givens records are NULL");
  } else {
    return fail(BGTQ_ERR_INVALID_ARG, "bad rotation kind %d", int(qz->rotation));
  }
  return BGTQ_OK;
}

}  // namespace

extern "C" {

const char* bgtq_status_string(bgtq_status s) {
  switch (s) {
    case BGTQ_OK: return "ok";
    case BGTQ_ERR_INVALID_ARG: return "invalid argument";
    case BGTQ_ERR_BUDGET: return "infeasible bit budget";
    case BGTQ_ERR_CAPACITY: return "cache capacity exceeded";
    case BGTQ_ERR_WORKSPACE: return "workspace too small";
    case BGTQ_ERR_UNSUPPORTED: return "unsupported configuration";
    case BGTQ_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* bgtq_last_error(void) { return g_last_error.c_str(); }

bgtq_status bgtq_init(void) { return ensure_init(); }

bgtq_status bgtq_set_option(bgtq_option option, int64_t value) {
  switch (option) {
    case BGTQ_OPT_DECODE_KERNEL:
      if (value < 0 || value > 2) return fail(BGTQ_ERR_INVALID_ARG, "decode kernel option must be 0, 1 or 2");
      g_decode_kernel = int(value);
      return BGTQ_OK;
    case BGTQ_OPT_STEP_WAIT_LIMIT:
      if (value < 0 || value > (int64_t(1) << 30)) return fail(BGTQ_ERR_INVALID_ARG, "wait limit must be 0..2^30");
      g_step_spin = int(value);
      return BGTQ_OK;
  }
  return fail(BGTQ_ERR_INVALID_ARG, "unknown option %d", int(option));
}

int64_t bgtq_get_option(bgtq_option option) {
  switch (option) {
    case BGTQ_OPT_DECODE_KERNEL: return g_decode_kernel;
    case BGTQ_OPT_STEP_WAIT_LIMIT: return g_step_spin;
  }
  return -1;
}

bgtq_status bgtq_codebook(int bits, float* thresholds, float* centroids, double* distortion) {
  if (bits < 0 || bits > BGTQ_MAX_BITS) return fail(BGTQ_ERR_INVALID_ARG, "bits must be 0..8");
  const Tables& t = host_tables();
  if (distortion) *distortion = t.dist[bits];
  if (bits == 0) return BGTQ_OK;
  if (thresholds) std::memcpy(thresholds, t.thr[bits - 1], sizeof(float) * ((1u << bits) - 1));
  if (centroids) std::memcpy(centroids, t.cen[bits - 1], sizeof(float) * (1u << bits));
  return BGTQ_OK;
}

size_t bgtq_rotation_bank_floats(int head_dim) {
  if (head_dim < 2 || head_dim > BGTQ_MAX_HEAD_DIM || head_dim % 2) return 0;
  return rot_bank_offset(head_dim + 2);
}

bgtq_status bgtq_transpose_rotations(const float* rot_bank, const float* rot_v, int head_dim, float* rot_bank_t,
                                     float* rot_v_t, bgtq_stream stream) {
  if (!rot_bank || !rot_v || !rot_bank_t || !rot_v_t) return fail(BGTQ_ERR_INVALID_ARG, "NULL rotation pointer");
  if (bgtq_rotation_bank_floats(head_dim) == 0) return fail(BGTQ_ERR_INVALID_ARG, "bad head_dim %d", head_dim);
  return hip_status(launch_transpose_rotations(rot_bank, rot_v, head_dim, rot_bank_t, rot_v_t,
                                               static_cast<hipStream_t>(stream)),
                    "rotation transpose launch");
}

size_t bgtq_cache_bytes(int batch, int n_kv_heads, int head_dim, int k_width_sum, int v_bits, int64_t capacity,
                        size_t* out4) {
  if (batch < 1 || n_kv_heads < 1 || !head_dim_ok(head_dim) || v_bits < 1 || v_bits > BGTQ_MAX_BITS ||
      k_width_sum < 0 || k_width_sum > BGTQ_MAX_BITS * (head_dim / 2) || capacity < kTile || capacity % kTile)
    return 0;
  const size_t heads = size_t(batch) * n_kv_heads, tiles = size_t(capacity / kTile);
  const size_t kc = heads * tiles * record_chunks(k_width_sum) * kTile * 16;
  const size_t kn = heads * tiles * kMaxGroups * kTile * 2;
  const size_t vc = heads * tiles * head_dim * 8 * v_bits;
  const size_t vn = heads * tiles * kTile * 2;
  if (out4) { out4[0] = kc; out4[1] = kn; out4[2] = vc; out4[3] = vn; }
  return kc + kn + vc + vn;
}

size_t bgtq_energy_workspace_bytes(int n_heads, int64_t n_tokens, int head_dim) {
  if (n_heads < 1 || n_tokens < 1 || !head_dim_ok(head_dim)) return 0;
  const int64_t chunks = (n_tokens + kEnergyChunk - 1) / kEnergyChunk;
  return size_t(n_heads) * size_t(chunks) * size_t(head_dim / 2) * sizeof(double);
}

bgtq_status bgtq_block_energy(const void* keys, bgtq_dtype dtype, int n_heads, int64_t n_tokens, int head_dim,
                              int64_t stride_head, int64_t stride_token, bgtq_pairing pairing, double* energy_out,
                              void* workspace, size_t workspace_bytes, bgtq_stream stream) {
  if (!keys || !energy_out) return fail(BGTQ_ERR_INVALID_ARG, "keys and energy_out must not be NULL");
  if (dtype != BGTQ_F32 && dtype != BGTQ_BF16) return fail(BGTQ_ERR_INVALID_ARG, "bad dtype");
  if (n_heads < 1 || n_tokens < 1) return fail(BGTQ_ERR_INVALID_ARG, "n_heads and n_tokens must be >= 1");
  if (!head_dim_ok(head_dim)) return fail(BGTQ_ERR_INVALID_ARG, "head_dim %d must be even, 2..256", head_dim);
  if (pairing != BGTQ_PAIR_HALF && pairing != BGTQ_PAIR_INTERLEAVED) return fail(BGTQ_ERR_INVALID_ARG, "bad pairing");
  if (stride_token < head_dim || (n_heads > 1 && stride_head < 1))
    return fail(BGTQ_ERR_INVALID_ARG, "strides must not overlap a key row");
  const size_t need = bgtq_energy_workspace_bytes(n_heads, n_tokens, head_dim);
  if (!workspace || workspace_bytes < need)
    return fail(BGTQ_ERR_WORKSPACE, "energy workspace needs %zu bytes", need);
  if (bgtq_status st = ensure_init(); st != BGTQ_OK) return st;
  return hip_status(launch_energy(keys, dtype, n_heads, n_tokens, head_dim, stride_head, stride_token, pairing,
                                  energy_out, static_cast<double*>(workspace), static_cast<hipStream_t>(stream)),
                    "block energy launch");
}

bgtq_status bgtq_allocate_bits(const double* energy, int n_heads, int head_dim, int k_width_sum, int b_min,
                               int b_max, bgtq_pairing pairing, uint8_t* widths_out, void* layouts_out,
                               bgtq_stream stream) {
  if (!energy || !widths_out || !layouts_out) return fail(BGTQ_ERR_INVALID_ARG, "NULL pointer");
  if (n_heads < 1) return fail(BGTQ_ERR_INVALID_ARG, "n_heads must be >= 1");
  if (!head_dim_ok(head_dim)) return fail(BGTQ_ERR_INVALID_ARG, "head_dim %d must be even, 2..256", head_dim);
  if (pairing != BGTQ_PAIR_HALF && pairing != BGTQ_PAIR_INTERLEAVED) return fail(BGTQ_ERR_INVALID_ARG, "bad pairing");
  const int n = head_dim / 2;
  if (b_min < 0 || b_max < b_min || b_max > BGTQ_MAX_BITS)
    return fail(BGTQ_ERR_BUDGET, "need 0 <= b_min <= b_max <= 8 (got %d, %d)", b_min, b_max);
  if (k_width_sum < n * b_min || k_width_sum > n * b_max)
    return fail(BGTQ_ERR_BUDGET, "k_width_sum %d outside [%d, %d]", k_width_sum, n * b_min, n * b_max);
  if (bgtq_status st = ensure_init(); st != BGTQ_OK) return st;
  return hip_status(launch_allocate(energy, n_heads, n, k_width_sum - n * b_min, b_min, b_max, pairing, widths_out,
                                    static_cast<HeadLayout*>(layouts_out), static_cast<hipStream_t>(stream)),
                    "allocate launch");
}

static bgtq_status prepare_append(const bgtq_quantizer* qz, const bgtq_cache* cache, int seq_begin, int n_seqs,
                                  const void* keys, const void* values, bgtq_dtype dtype, int64_t n_new,
                                  int64_t stride_seq, int64_t stride_head, int64_t stride_token, AppendArgs& a) {
  if (bgtq_status st = check_cache(cache, true); st != BGTQ_OK) return st;
  if (bgtq_status st = check_quantizer(qz); st != BGTQ_OK) return st;
  if (qz->head_dim != cache->head_dim) return fail(BGTQ_ERR_INVALID_ARG, "quantizer head_dim != cache head_dim");
  if (!keys || !values) return fail(BGTQ_ERR_INVALID_ARG, "keys and values must not be NULL");
  if (dtype != BGTQ_F32 && dtype != BGTQ_BF16) return fail(BGTQ_ERR_INVALID_ARG, "bad dtype");
  if (n_seqs < 1 || seq_begin < 0 || seq_begin + n_seqs > cache->batch)
    return fail(BGTQ_ERR_INVALID_ARG, "sequence range [%d, %d) outside batch %d", seq_begin, seq_begin + n_seqs,
                cache->batch);
  if (n_new < 1) return fail(BGTQ_ERR_INVALID_ARG, "n_new must be >= 1");
  if (n_new > cache->capacity) return fail(BGTQ_ERR_CAPACITY, "n_new %lld exceeds capacity %lld",
                                           (long long)n_new, (long long)cache->capacity);
  if (stride_token < cache->head_dim || stride_head < 1 || stride_seq < 1)
    return fail(BGTQ_ERR_INVALID_ARG, "strides must be positive and not overlap a row");
  a = AppendArgs{};
  a.advance = 1;
  a.rot_bank = qz->rot_bank;
  a.rot_v = qz->rot_v;
  a.rot_bank_t = qz->rot_bank_t;
  a.rot_v_t = qz->rot_v_t;
  a.keys = keys;
  a.values = values;
  a.stride_seq = stride_seq;
  a.stride_head = stride_head;
  a.stride_token = stride_token;
  a.k_codes = cache->k_codes;
  a.k_norms = cache->k_norms;
  a.v_codes = cache->v_codes;
  a.v_norms = cache->v_norms;
  a.lengths = cache->lengths;
  a.layouts = static_cast<const HeadLayout*>(cache->layouts);
  a.status = cache->status;
  a.capacity = cache->capacity;
  a.n_new = n_new;
  a.seq_begin = seq_begin;
  a.n_kv_heads = cache->n_kv_heads;
  a.d = cache->head_dim;
  a.v_bits = cache->v_bits;
  a.chunks = record_chunks(cache->k_width_sum);
  a.window = cache->window;
  a.k_window = cache->window > 0 ? cache->k_window : nullptr;
  a.givens = qz->rotation == BGTQ_ROT_GIVENS ? reinterpret_cast<const uint4*>(qz->givens) : nullptr;
  return BGTQ_OK;
}

bgtq_status bgtq_quantize_append(const bgtq_quantizer* qz, const bgtq_cache* cache, int seq_begin, int n_seqs,
                                 const void* keys, const void* values, bgtq_dtype dtype, int64_t n_new,
                                 int64_t stride_seq, int64_t stride_head, int64_t stride_token, bgtq_stream stream) {
  AppendArgs a;
  if (bgtq_status st = prepare_append(qz, cache, seq_begin, n_seqs, keys, values, dtype, n_new, stride_seq,
                                      stride_head, stride_token, a);
      st != BGTQ_OK)
    return st;
  if (bgtq_status st = ensure_init(); st != BGTQ_OK) return st;
  return hip_status(launch_append(a, dtype, n_seqs, static_cast<hipStream_t>(stream)), "quantize-append launch");
}

size_t bgtq_prefill_workspace_bytes(int n_kv_heads, int64_t n_tokens, int head_dim) {
  return bgtq_energy_workspace_bytes(n_kv_heads, n_tokens, head_dim);
}

bgtq_status bgtq_prefill(const bgtq_quantizer* qz, const bgtq_cache* cache, int seq, const void* keys,
                         const void* values, bgtq_dtype dtype, int64_t n_tokens, int64_t stride_head,
                         int64_t stride_token, int b_min, int b_max, double* energy_out, void* workspace,
                         size_t workspace_bytes, bgtq_stream stream) {
  if (bgtq_status st = check_cache(cache, true); st != BGTQ_OK) return st;
  if (seq < 0 || seq >= cache->batch) return fail(BGTQ_ERR_INVALID_ARG, "sequence %d outside batch %d", seq, cache->batch);
  if (!cache->widths) return fail(BGTQ_ERR_INVALID_ARG, "widths is NULL");
  const int d = cache->head_dim, n = d / 2;
  if (b_min < 0 || b_max < b_min || b_max > BGTQ_MAX_BITS)
    return fail(BGTQ_ERR_BUDGET, "need 0 <= b_min <= b_max <= 8 (got %d, %d)", b_min, b_max);
  if (cache->k_width_sum < n * b_min || cache->k_width_sum > n * b_max)
    return fail(BGTQ_ERR_BUDGET, "k_width_sum %d outside [%d, %d]", cache->k_width_sum, n * b_min, n * b_max);
  if (n_tokens < 1) return fail(BGTQ_ERR_INVALID_ARG, "n_tokens must be >= 1");
  if (cache->n_kv_heads > 1 && stride_head < 1) return fail(BGTQ_ERR_INVALID_ARG, "stride_head must be >= 1");
  AppendArgs aa;
  if (bgtq_status st = prepare_append(qz, cache, seq, 1, keys, values, dtype, n_tokens,
                                      stride_head * cache->n_kv_heads > 0 ? stride_head * cache->n_kv_heads : 1,
                                      stride_head > 0 ? stride_head : 1, stride_token, aa);
      st != BGTQ_OK)
    return st;
  const size_t need = bgtq_prefill_workspace_bytes(cache->n_kv_heads, n_tokens, d);
  if (!workspace || workspace_bytes < need) return fail(BGTQ_ERR_WORKSPACE, "prefill workspace needs %zu bytes", need);
  if (bgtq_status st = ensure_init(); st != BGTQ_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t reg = size_t(seq) * cache->n_kv_heads;
  if (bgtq_status st = hip_status(
          launch_prefill_alloc(keys, dtype, cache->n_kv_heads, n_tokens, d, stride_head, stride_token, cache->pairing,
                               static_cast<double*>(workspace), cache->k_width_sum - n * b_min, b_min, b_max,
                               energy_out, cache->widths + reg * n, static_cast<HeadLayout*>(cache->layouts) + reg, s),
          "prefill energy/allocation launch");
      st != BGTQ_OK)
    return st;
  return hip_status(launch_append(aa, dtype, 1, s), "prefill quantize-append launch");
}

size_t bgtq_decode_workspace_bytes(int batch, int n_q_heads, int n_kv_heads, int head_dim, int64_t capacity) {
  if (batch < 1 || n_q_heads < 1 || n_kv_heads < 1 || !head_dim_ok(head_dim) || capacity < kTile) return 0;
  // an upper bound of every pass's split count (the streamed matrix-core pass, the other
  // matrix-core pass with its window splits, the vector-ALU pass)
  const int base = std::max(std::max(decode_splits(batch, n_kv_heads, capacity, true),
                                     decode_splits(batch, n_kv_heads, capacity, false)),
                            decode_stream_splits(batch, n_kv_heads));
  const int splits = base + kMaxWindowSplits;
  const size_t part = align256(size_t(batch) * n_q_heads * splits * head_dim * 4) +
                      align256(size_t(batch) * n_q_heads * splits * 8);
  return align256(decode_qrot_bytes(batch, n_kv_heads, head_dim)) + part +
         align256(decode_step_bytes(batch, n_kv_heads));
}

static bgtq_status prepare_decode(const bgtq_quantizer* qz, const bgtq_cache* cache, int n_q_heads, const void* q,
                                  bgtq_dtype q_dtype, const int64_t* q_pos, double rope_theta, float softmax_scale,
                                  float* out, float* logits_out, void* workspace, size_t workspace_bytes,
                                  DecodeArgs& a) {
  if (bgtq_status st = check_cache(cache, true); st != BGTQ_OK) return st;
  if (bgtq_status st = check_quantizer(qz); st != BGTQ_OK) return st;
  if (qz->head_dim != cache->head_dim) return fail(BGTQ_ERR_INVALID_ARG, "quantizer head_dim != cache head_dim");
  if (!q || !out) return fail(BGTQ_ERR_INVALID_ARG, "q and out must not be NULL");
  if (q_dtype != BGTQ_F32 && q_dtype != BGTQ_BF16) return fail(BGTQ_ERR_INVALID_ARG, "bad q dtype");
  if (n_q_heads < cache->n_kv_heads || n_q_heads % cache->n_kv_heads)
    return fail(BGTQ_ERR_INVALID_ARG, "n_q_heads %d must be a multiple of n_kv_heads %d", n_q_heads,
                cache->n_kv_heads);
  const int group = n_q_heads / cache->n_kv_heads;
  if (group > BGTQ_MAX_GROUP) return fail(BGTQ_ERR_UNSUPPORTED, "group size %d > %d", group, BGTQ_MAX_GROUP);
  const int d = cache->head_dim;
  if (d != 64 && d != 128 && d != 256) return fail(BGTQ_ERR_UNSUPPORTED, "decode is built for head_dim 64/128/256");
  if (!(softmax_scale > 0.0f)) return fail(BGTQ_ERR_INVALID_ARG, "softmax_scale must be > 0");
  const size_t need = bgtq_decode_workspace_bytes(cache->batch, n_q_heads, cache->n_kv_heads, d, cache->capacity);
  if (!workspace || workspace_bytes < need)
    return fail(BGTQ_ERR_WORKSPACE, "decode workspace needs %zu bytes", need);
  a = DecodeArgs{};
  a.rot_bank = qz->rot_bank;
  a.rot_v = qz->rot_v;
  a.rot_bank_t = qz->rot_bank_t;
  a.q = q;
  a.q_pos = q_pos;
  a.k_codes = cache->k_codes;
  a.k_norms = cache->k_norms;
  a.v_codes = cache->v_codes;
  a.v_norms = cache->v_norms;
  a.lengths = cache->lengths;
  a.layouts = static_cast<const HeadLayout*>(cache->layouts);
  a.out = out;
  a.logits = logits_out;
  a.use_mfma = group <= 8 && g_decode_kernel != 1;
  if (cache->window > 0 && !a.use_mfma)
    return fail(BGTQ_ERR_UNSUPPORTED, "the recent-key window is built on the matrix-core decode (group size <= 8)");
  a.window = cache->window;
  a.k_window = cache->window > 0 ? cache->k_window : nullptr;
  // the window's splits come out of the same workgroup budget (a grid that fits the GPU at
  // once), the packed keys keep at least one split
  a.n_wsplit = window_splits(cache->window);
  a.use_stream = a.use_mfma && g_decode_kernel != 2 && cache->window == 0 &&
                 decode_stream_fits(d, record_chunks(cache->k_width_sum), cache->v_bits);
  if (a.use_stream) {
    a.n_split = decode_stream_splits(cache->batch, cache->n_kv_heads);
    a.stream_whole_tiles = decode_stream_whole_tiles(cache->batch, cache->n_kv_heads) ? 1 : 0;
  } else {
    const int base = decode_splits(cache->batch, cache->n_kv_heads, cache->capacity, a.use_mfma);
    // the matrix-core pass leaves one workgroup of every (sequence, KV head) to a decode step's
    // append role, so that a step and a decode call split the tokens alike
    const int packed = base - a.n_wsplit - (a.use_mfma ? 1 : 0);
    a.n_split = (packed > 1 ? packed : 1) + a.n_wsplit;
  }
  // the partial results of this split count must fit the workspace layout (the size function
  // bounds every pass's count)
  const size_t used = align256(decode_qrot_bytes(cache->batch, cache->n_kv_heads, d)) +
                      align256(size_t(cache->batch) * n_q_heads * a.n_split * d * 4) +
                      align256(size_t(cache->batch) * n_q_heads * a.n_split * 8) +
                      align256(decode_step_bytes(cache->batch, cache->n_kv_heads));
  if (used > need) return fail(BGTQ_ERR_WORKSPACE, "internal: %d splits need %zu workspace bytes, sized %zu",
                               a.n_split, used, need);
  char* ws = static_cast<char*>(workspace);
  const size_t qrot_b = align256(decode_qrot_bytes(cache->batch, cache->n_kv_heads, d));
  a.qrot = reinterpret_cast<float*>(ws);
  a.partial = reinterpret_cast<float*>(ws + qrot_b);
  a.part_ml = reinterpret_cast<float2*>(ws + qrot_b + align256(size_t(cache->batch) * n_q_heads * a.n_split * d * 4));
  a.givens = qz->rotation == BGTQ_ROT_GIVENS ? reinterpret_cast<const uint4*>(qz->givens) : nullptr;
  a.rope_theta = rope_theta;
  for (int j = 0; j < d / 2; ++j) a.inv_freq[j] = rope_theta > 0.0 ? std::pow(rope_theta, -2.0 * j / d) : 0.0;
  a.scale = softmax_scale;
  a.capacity = cache->capacity;
  a.batch = cache->batch;
  a.n_q = n_q_heads;
  a.n_kv = cache->n_kv_heads;
  a.group = group;
  a.d = d;
  a.v_bits = cache->v_bits;
  a.chunks = record_chunks(cache->k_width_sum);
  a.pairing = cache->pairing;
  return BGTQ_OK;
}

bgtq_status bgtq_decode_attention(const bgtq_quantizer* qz, const bgtq_cache* cache, int n_q_heads, const void* q,
                                  bgtq_dtype q_dtype, const int64_t* q_pos, double rope_theta, float softmax_scale,
                                  float* out, float* logits_out, void* workspace, size_t workspace_bytes,
                                  bgtq_stream stream) {
  DecodeArgs a;
  if (bgtq_status st = prepare_decode(qz, cache, n_q_heads, q, q_dtype, q_pos, rope_theta, softmax_scale, out,
                                      logits_out, workspace, workspace_bytes, a);
      st != BGTQ_OK)
    return st;
  if (bgtq_status st = ensure_init(); st != BGTQ_OK) return st;
  return hip_status(launch_decode(a, q_dtype, static_cast<hipStream_t>(stream)), "decode launch");
}

// a decode step on a given workspace; with noalloc, the workspace is the current device's
// scratch array (looked up after the arguments are validated) and its step flags are cleared
// first
static bgtq_status decode_step(const bgtq_quantizer* qz, const bgtq_cache* cache, int n_q_heads, const void* q,
                               bgtq_dtype q_dtype, const void* keys, const void* values, bgtq_dtype kv_dtype,
                               int64_t stride_seq, int64_t stride_head, double rope_theta, float softmax_scale,
                               float* out, float* logits_out, void* workspace, size_t workspace_bytes,
                               hipStream_t s, bool noalloc) {
  if (bgtq_status st = check_cache(cache, true); st != BGTQ_OK) return st;
  if (noalloc) {
    const size_t need = bgtq_decode_workspace_bytes(cache->batch, n_q_heads, cache->n_kv_heads, cache->head_dim,
                                                    cache->capacity);
    if (need > BGTQ_NOALLOC_SCRATCH_BYTES)
      return fail(BGTQ_ERR_WORKSPACE, "this cache needs %zu bytes of decode workspace; the allocation-free "
                  "scratch holds %u (use bgtq_decode_step with a workspace)", need, BGTQ_NOALLOC_SCRATCH_BYTES);
    // the arguments are validated against a stand-in address; the scratch's own address is
    // looked up once they pass (the lookup initialises the device)
    workspace = reinterpret_cast<void*>(uintptr_t(256));
    workspace_bytes = BGTQ_NOALLOC_SCRATCH_BYTES;
  }
  AppendArgs aa;
  if (bgtq_status st = prepare_append(qz, cache, 0, cache->batch, keys, values, kv_dtype, 1, stride_seq, stride_head,
                                      cache->head_dim, aa);
      st != BGTQ_OK)
    return st;
  DecodeArgs da;
  if (bgtq_status st = prepare_decode(qz, cache, n_q_heads, q, q_dtype, nullptr, rope_theta, softmax_scale, out,
                                      logits_out, workspace, workspace_bytes, da);
      st != BGTQ_OK)
    return st;
  if (bgtq_status st = ensure_init(); st != BGTQ_OK) return st;
  if (noalloc) {
    int dev = 0;
    if (hipError_t e = hipGetDevice(&dev); e != hipSuccess) return hip_status(e, "hipGetDevice");
    workspace = g_scratch[dev];
    if (bgtq_status st = prepare_decode(qz, cache, n_q_heads, q, q_dtype, nullptr, rope_theta, softmax_scale, out,
                                        logits_out, workspace, workspace_bytes, da);
        st != BGTQ_OK)
      return st;
  }
  const size_t need = bgtq_decode_workspace_bytes(cache->batch, n_q_heads, cache->n_kv_heads, cache->head_dim,
                                                  cache->capacity);
  int32_t* flags = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + need -
                                              align256(decode_step_bytes(cache->batch, cache->n_kv_heads)));
  if (noalloc) {   // the scratch keeps the last call's contents: the flags must start at zero
    if (bgtq_status st = hip_status(launch_clear_flags(flags, cache->batch * cache->n_kv_heads, s),
                                    "decode-step flag clear launch");
        st != BGTQ_OK)
      return st;
  }
  if (!da.use_mfma) {   // vector-ALU path: the two calls in sequence
    if (bgtq_status st = hip_status(launch_append(aa, kv_dtype, cache->batch, s), "decode-step append launch");
        st != BGTQ_OK)
      return st;
    return hip_status(launch_decode(da, q_dtype, s), "decode-step attention launch");
  }
  aa.advance = 0;
  da.step = 1;
  // the wait of the split that reads the new token's tile is bounded (about 0.2 s at most by
  // default); the option BGTQ_OPT_STEP_WAIT_LIMIT sets the bound (0: no wait), so that the
  // report of a wait that gave up can be exercised
  da.step_spin = g_step_spin;
  da.step_flag = flags;
  return hip_status(launch_decode_step(aa, da, kv_dtype, q_dtype, s), "decode-step launch");
}

bgtq_status bgtq_decode_step(const bgtq_quantizer* qz, const bgtq_cache* cache, int n_q_heads, const void* q,
                             bgtq_dtype q_dtype, const void* keys, const void* values, bgtq_dtype kv_dtype,
                             int64_t stride_seq, int64_t stride_head, double rope_theta, float softmax_scale,
                             float* out, float* logits_out, void* workspace, size_t workspace_bytes,
                             bgtq_stream stream) {
  return decode_step(qz, cache, n_q_heads, q, q_dtype, keys, values, kv_dtype, stride_seq, stride_head, rope_theta,
                     softmax_scale, out, logits_out, workspace, workspace_bytes, static_cast<hipStream_t>(stream),
                     false);
}

bgtq_status bgtq_decode_step_noalloc(const bgtq_quantizer* qz, const bgtq_cache* cache, int n_q_heads,
                                     const void* q, bgtq_dtype q_dtype, const void* keys, const void* values,
                                     bgtq_dtype kv_dtype, int64_t stride_seq, int64_t stride_head,
                                     double rope_theta, float softmax_scale, float* out, float* logits_out,
                                     bgtq_stream stream) {
  return decode_step(qz, cache, n_q_heads, q, q_dtype, keys, values, kv_dtype, stride_seq, stride_head, rope_theta,
                     softmax_scale, out, logits_out, nullptr, 0, static_cast<hipStream_t>(stream), true);
}

size_t bgtq_logit_error_workspace_bytes(int batch, int n_q_heads, int64_t capacity) {
  if (batch < 1 || n_q_heads < 1 || capacity < 1) return 0;
  return align256(size_t(batch) * n_q_heads * size_t((capacity + kErrChunk - 1) / kErrChunk) * 8);
}

bgtq_status bgtq_logit_error(const void* q, bgtq_dtype q_dtype, const int64_t* q_pos, const void* keys,
                             bgtq_dtype k_dtype, int batch, int n_q_heads, int n_kv_heads, int head_dim,
                             int64_t stride_seq, int64_t stride_head, int64_t stride_token,
                             const int32_t* lengths, int64_t capacity, bgtq_pairing pairing,
                             double rope_theta, float softmax_scale, const float* logits, double* mae_out,
                             void* workspace, size_t workspace_bytes, bgtq_stream stream) {
  if (!q || !keys || !lengths || !logits || !mae_out)
    return fail(BGTQ_ERR_INVALID_ARG, "q, keys, lengths, logits and mae_out must not be NULL");
  if (q_dtype != BGTQ_F32 && q_dtype != BGTQ_BF16) return fail(BGTQ_ERR_INVALID_ARG, "bad q dtype");
  if (k_dtype != BGTQ_F32 && k_dtype != BGTQ_BF16) return fail(BGTQ_ERR_INVALID_ARG, "bad key dtype");
  if (pairing != BGTQ_PAIR_HALF && pairing != BGTQ_PAIR_INTERLEAVED) return fail(BGTQ_ERR_INVALID_ARG, "bad pairing");
  if (batch < 1 || n_kv_heads < 1) return fail(BGTQ_ERR_INVALID_ARG, "batch and n_kv_heads must be >= 1");
  if (n_q_heads < n_kv_heads || n_q_heads % n_kv_heads)
    return fail(BGTQ_ERR_INVALID_ARG, "n_q_heads %d must be a multiple of n_kv_heads %d", n_q_heads, n_kv_heads);
  const int group = n_q_heads / n_kv_heads;
  if (group > BGTQ_MAX_GROUP) return fail(BGTQ_ERR_UNSUPPORTED, "group size %d > %d", group, BGTQ_MAX_GROUP);
  if (head_dim != 64 && head_dim != 128 && head_dim != 256)
    return fail(BGTQ_ERR_UNSUPPORTED, "the logit error is built for head_dim 64/128/256");
  if (capacity < 1) return fail(BGTQ_ERR_INVALID_ARG, "capacity must be >= 1");
  if (capacity % 4) return fail(BGTQ_ERR_INVALID_ARG, "capacity must be a multiple of 4");
  if (stride_seq < 0 || stride_head < 0 || stride_token < head_dim || stride_seq % 4 || stride_head % 4 ||
      stride_token % 4)
    return fail(BGTQ_ERR_INVALID_ARG, "key strides must be multiples of 4 with stride_token >= head_dim");
  const uintptr_t kal = k_dtype == BGTQ_F32 ? 16 : 8;
  if (reinterpret_cast<uintptr_t>(keys) % kal || reinterpret_cast<uintptr_t>(logits) % 16)
    return fail(BGTQ_ERR_INVALID_ARG, "keys or logits misaligned");
  if (!(softmax_scale > 0.0f)) return fail(BGTQ_ERR_INVALID_ARG, "softmax_scale must be > 0");
  const size_t need = bgtq_logit_error_workspace_bytes(batch, n_q_heads, capacity);
  if (!workspace || workspace_bytes < need) return fail(BGTQ_ERR_WORKSPACE, "logit-error workspace needs %zu bytes", need);
  LogitErrArgs a{};
  a.q = q;
  a.q_pos = q_pos;
  a.keys = keys;
  a.stride_seq = stride_seq;
  a.stride_head = stride_head;
  a.stride_token = stride_token;
  a.lengths = lengths;
  a.logits = logits;
  a.partial = static_cast<double*>(workspace);
  a.mae = mae_out;
  a.rope_theta = rope_theta;
  for (int j = 0; j < head_dim / 2; ++j) a.inv_freq[j] = rope_theta > 0.0 ? std::pow(rope_theta, -2.0 * j / head_dim) : 0.0;
  a.scale = softmax_scale;
  a.capacity = capacity;
  a.batch = batch;
  a.n_q = n_q_heads;
  a.n_kv = n_kv_heads;
  a.group = group;
  a.d = head_dim;
  a.pairing = pairing;
  a.n_chunk = int((capacity + kErrChunk - 1) / kErrChunk);
  return hip_status(launch_logit_error(a, k_dtype, q_dtype, static_cast<hipStream_t>(stream)), "logit-error launch");
}

}  // extern "C"
