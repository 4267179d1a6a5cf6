// Host side of the C ABI declared in include/inkling_rel_attn.h: argument
// validation (host-visible values only, no device access), the split-count
// heuristic, workspace sizing, the device check and the kernel launches.
//
// The device check mirrors the fail-fast guard of the vLLM page (section
// "Purpose" and "Changes"): an unsupported GPU is rejected up front with a
// message naming the device, instead of failing inside a kernel later.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <initializer_list>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "inkling_rel_attn.h"
#include "launch.hpp"

using namespace ira;

namespace {

size_t dtype_size(int32_t dtype) { return dtype == INKLING_DTYPE_BF16 ? 2 : 4; }

// Validation shared by both entry points.  Never touches device memory.
inkling_status_t check_dims(const inkling_rel_attn_dims_t* d) {
  if (d == nullptr) return INKLING_ERR_INVALID_ARGUMENT;
  if (d->num_seqs < 0 || d->num_q_heads <= 0 || d->num_kv_heads <= 0 ||
      d->num_blocks <= 0 || d->max_blocks_per_seq <= 0 || d->rel_len <= 0 ||
      d->total_q < 0 || d->max_q_len < 0 || d->max_seq_len < 0)
    return INKLING_ERR_INVALID_ARGUMENT;
  if (d->num_q_heads % d->num_kv_heads != 0) return INKLING_ERR_INVALID_ARGUMENT;
  // Sequences and KV heads index grid dimensions limited to 65535.
  if (d->num_seqs > 65535 || d->num_kv_heads > 65535) return INKLING_ERR_UNSUPPORTED;
  if (d->dtype != INKLING_DTYPE_BF16 && d->dtype != INKLING_DTYPE_FP32)
    return INKLING_ERR_UNSUPPORTED;
  if (d->head_dim != 64 && d->head_dim != 128) return INKLING_ERR_UNSUPPORTED;
  if (d->block_size != 16) return INKLING_ERR_UNSUPPORTED;
  if (d->num_q_heads / d->num_kv_heads > kMaxGroup) return INKLING_ERR_UNSUPPORTED;
  if ((d->rel_len * dtype_size(d->dtype)) % 16 != 0) return INKLING_ERR_UNSUPPORTED;
  if (d->max_q_len > d->max_seq_len) return INKLING_ERR_INVALID_ARGUMENT;
  if ((int64_t)d->max_blocks_per_seq * d->block_size < d->max_seq_len)
    return INKLING_ERR_INVALID_ARGUMENT;
  return INKLING_OK;
}

int device_cus(int32_t device) {
  int cus = 0;
  if (device >= 0 &&
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) == hipSuccess &&
      cus > 0)
    return cus;
  (void)hipGetLastError();
  return 256;
}

// 32-key tiles a decode wave may have to cover for one sequence: the visible
// keys (the window on local layers, the whole context on global ones) plus
// up to 15 keys of alignment to the first page.
int64_t decode_max_tiles(const inkling_rel_attn_dims_t* d, int32_t window) {
  const int64_t keys = window > 0 ? std::min<int64_t>(window, d->max_seq_len)
                                  : (int64_t)d->max_seq_len;
  return std::max<int64_t>(1, (keys + 15 + kDecodeKeys - 1) / kDecodeKeys);
}

// Tiles per split for a given split count: sequence b then uses
// ceil(tiles_b / chunk) <= num_splits splits.
int32_t decode_chunk_tiles(const inkling_rel_attn_dims_t* d, int32_t window, int32_t splits) {
  const int64_t t = decode_max_tiles(d, window);
  return (int32_t)((t + splits - 1) / splits);
}

int32_t splits_for(const inkling_rel_attn_dims_t* d, int32_t window, int cus) {
  const int64_t units = (int64_t)d->num_seqs * d->num_kv_heads;
  if (units <= 0) return 1;
  // One wave per (sequence, KV head, split); aim for one wave per SIMD of
  // the device.  Long key ranges keep at least 8 tiles (256 keys) in every
  // split; short ones (a local window) go down to 2 tiles, since there the
  // per-split chain, not the merge, sets the latency (measured at 1-16
  // sequences of a 512-key window: 8 splits of 3 tiles beat 2 of 9 by 30%).
  const int64_t tiles = decode_max_tiles(d, window);
  const int64_t want = ((int64_t)kDecodeWavesPerCU * cus + units - 1) / units;
  const int64_t cap = std::max<int64_t>(1, tiles >= 64 ? tiles / 8 : tiles / 2);
  int64_t s = std::min<int64_t>(want, cap);
  s = std::max<int64_t>(1, std::min<int64_t>(s, kMaxSplits));
  return (int32_t)s;
}

// Tensors are read and written in 16-byte vectors.
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }
bool all_aligned16(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (p != nullptr && !aligned16(p)) return false;
  return true;
}

size_t workspace_for(const inkling_rel_attn_dims_t* d, int32_t splits) {
  if (splits <= 1) return 0;
  const size_t rows = (size_t)d->num_seqs * d->num_q_heads;
  const size_t o = (size_t)splits * rows * d->head_dim * sizeof(float);
  const size_t l = (size_t)splits * rows * sizeof(float);
  return ((o + 255) & ~(size_t)255) + l;
}

}  // namespace

extern "C" {

const char* inkling_rel_attn_status_string(inkling_status_t s) {
  switch (s) {
    case INKLING_OK: return "ok";
    case INKLING_ERR_INVALID_ARGUMENT: return "invalid argument";
    case INKLING_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case INKLING_ERR_UNSUPPORTED_DEVICE: return "unsupported device (needs gfx950)";
    case INKLING_ERR_NO_DEVICE: return "no HIP device";
    case INKLING_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case INKLING_ERR_LAUNCH: return "kernel launch failed";
  }
  return "unknown status";
}

inkling_status_t inkling_rel_attn_check_device(int32_t device, char* msg, size_t msg_len) {
  auto say = [&](const char* text) {
    if (msg != nullptr && msg_len > 0) {
      std::snprintf(msg, msg_len, "%s", text);
    }
  };
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || count <= 0) {
    (void)hipGetLastError();
    say("no HIP device is visible");
    return INKLING_ERR_NO_DEVICE;
  }
  if (device < 0 || device >= count) {
    char buf[128];
    std::snprintf(buf, sizeof buf, "device %d does not exist (%d visible)", device, count);
    say(buf);
    return INKLING_ERR_INVALID_ARGUMENT;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, device) != hipSuccess) {
    (void)hipGetLastError();
    say("device properties unavailable");
    return INKLING_ERR_NO_DEVICE;
  }
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) {
    char buf[512];
    std::snprintf(buf, sizeof buf,
                  "device %d (%s, %s) is not supported: this library is built for gfx950 (MI355X)",
                  device, prop.name, prop.gcnArchName);
    say(buf);
    return INKLING_ERR_UNSUPPORTED_DEVICE;
  }
  say("ok");
  return INKLING_OK;
}

int32_t inkling_rel_attn_num_splits(const inkling_rel_attn_dims_t* dims, int32_t window,
                                    int32_t device) {
  if (dims == nullptr || dims->num_seqs <= 0 || dims->num_kv_heads <= 0) return 1;
  return splits_for(dims, window, device_cus(device));
}

size_t inkling_rel_attn_decode_workspace_bytes(const inkling_rel_attn_dims_t* dims,
                                               int32_t window, int32_t num_splits) {
  if (dims == nullptr || num_splits < 0 || num_splits > kMaxSplits) return 0;
  if (num_splits == 0) num_splits = inkling_rel_attn_num_splits(dims, window, 0);
  return workspace_for(dims, num_splits);
}

}  // extern "C"

namespace {

inkling_status_t prefill_impl(const void* q, const void* k_new, const void* v_new,
                              const void* k_cache, const void* v_cache,
                              const int32_t* block_table, const int32_t* seq_lens,
                              const int32_t* cu_q_lens, const void* rel_logits, int32_t window,
                              float scale, void* out, const inkling_rel_attn_dims_t* dims,
                              void* stream) {
  inkling_status_t st = check_dims(dims);
  if (st != INKLING_OK) return st;
  if (!std::isfinite(scale)) return INKLING_ERR_INVALID_ARGUMENT;
  if (dims->num_seqs == 0 || dims->total_q == 0 || dims->max_q_len == 0) return INKLING_OK;
  if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !cu_q_lens || !rel_logits || !out)
    return INKLING_ERR_INVALID_ARGUMENT;
  if (!all_aligned16({q, k_cache, v_cache, rel_logits, out, k_new, v_new}))
    return INKLING_ERR_INVALID_ARGUMENT;

  PrefillParams p{};
  p.q = q;
  p.k = k_cache;
  p.v = v_cache;
  p.block_table = block_table;
  p.seq_lens = seq_lens;
  p.cu_q_lens = cu_q_lens;
  p.rel = rel_logits;
  p.out = out;
  p.k_new = k_new;
  p.v_new = v_new;
  p.hq = dims->num_q_heads;
  p.hkv = dims->num_kv_heads;
  p.group = dims->num_q_heads / dims->num_kv_heads;
  p.num_blocks = dims->num_blocks;
  p.max_blocks = dims->max_blocks_per_seq;
  p.rel_len = dims->rel_len;
  p.window = window;
  p.total_q = dims->total_q;
  p.scale = scale;
  // Query tokens per workgroup: G heads x bq tokens fill the 4 waves' 128
  // MFMA columns.
  p.bq = 128 / p.group;
  const int waves = kPrefillWaves;
  const size_t esz = dtype_size(dims->dtype);
  const int vec = (int)(16 / esz);
  p.sb = std::min(dims->rel_len, kPrefillKeys + vec);
  int row_dw = (int)((p.sb * esz + 3) / 4);
  if ((row_dw & 1) == 0) row_dw += 1;  // odd dword pitch spreads LDS banks
  p.sb_pitch = row_dw * 4;
  p.nqb = (dims->max_q_len + p.bq - 1) / p.bq;
  p.num_seqs = dims->num_seqs;
  // Pages a workgroup's key range can touch (the generic kernel's LDS page
  // table; the bf16 kernel reads page ids with scalar loads instead).
  const int64_t span = window > 0 ? (int64_t)p.bq + window - 1 : (int64_t)dims->max_seq_len;
  p.pid_cap = (int32_t)std::min<int64_t>(dims->max_blocks_per_seq, (span + 15) / 16 + 2);
  // bf16 with head_dim 128 runs the specialised kernel (with or without the
  // fused append).
  const bool bf16_fast = dims->dtype == INKLING_DTYPE_BF16 && dims->head_dim == 128;
  if ((bf16_fast ? prefill_bf16_lds_bytes()
                 : prefill_lds_bytes(dims->dtype, dims->head_dim, waves, p.sb_pitch, p.pid_cap)) >
      160 * 1024)
    return INKLING_ERR_UNSUPPORTED;
  // 32-bit buffer offsets: one page, and the bias rows of one query block.
  if ((int64_t)16 * dims->num_kv_heads * dims->head_dim * (int64_t)esz >= (1LL << 31) ||
      (int64_t)p.bq * dims->num_q_heads * dims->rel_len * (int64_t)esz >= (1LL << 31))
    return INKLING_ERR_UNSUPPORTED;
  if ((int64_t)p.nqb * dims->num_seqs * dims->num_kv_heads >= (1LL << 31) ||
      ((int64_t)dims->total_q / p.bq + dims->num_seqs) * dims->num_kv_heads >= (1LL << 31))
    return INKLING_ERR_UNSUPPORTED;
  const hipError_t e = bf16_fast ? launch_prefill_bf16(p, static_cast<hipStream_t>(stream))
                                 : launch_prefill(p, dims->dtype, dims->head_dim,
                                                  static_cast<hipStream_t>(stream));
  return e == hipSuccess ? INKLING_OK : INKLING_ERR_LAUNCH;
}


inkling_status_t decode_impl(const void* q, const void* k_new, const void* v_new,
                             const void* k_cache, const void* v_cache,
                             const int32_t* block_table, const int32_t* seq_lens,
                             const void* rel_logits, int32_t window, float scale,
                             int32_t num_splits, void* workspace, size_t workspace_bytes,
                             void* out, const inkling_rel_attn_dims_t* dims, void* stream) {
  inkling_status_t st = check_dims(dims);
  if (st != INKLING_OK) return st;
  if (!std::isfinite(scale)) return INKLING_ERR_INVALID_ARGUMENT;
  if (num_splits < 0 || num_splits > kMaxSplits) return INKLING_ERR_INVALID_ARGUMENT;
  if (dims->total_q != dims->num_seqs) return INKLING_ERR_INVALID_ARGUMENT;
  if (dims->num_seqs == 0) return INKLING_OK;
  if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !rel_logits || !out)
    return INKLING_ERR_INVALID_ARGUMENT;
  if (!all_aligned16({q, k_cache, v_cache, rel_logits, out, k_new, v_new}))
    return INKLING_ERR_INVALID_ARGUMENT;
  int dev = 0;
  if (num_splits == 0) {
    if (hipGetDevice(&dev) != hipSuccess) {
      (void)hipGetLastError();
      dev = -1;
    }
    num_splits = splits_for(dims, window, device_cus(dev));
  }
  const size_t need = workspace_for(dims, num_splits);
  if (need > 0) {
    if (workspace == nullptr || workspace_bytes < need) return INKLING_ERR_WORKSPACE_TOO_SMALL;
    if ((reinterpret_cast<uintptr_t>(workspace) & 15) != 0) return INKLING_ERR_INVALID_ARGUMENT;
  }

  DecodeParams p{};
  p.q = q;
  p.k = k_cache;
  p.v = v_cache;
  p.k_new = k_new;
  p.v_new = v_new;
  p.block_table = block_table;
  p.seq_lens = seq_lens;
  p.rel = rel_logits;
  p.out = out;
  const size_t rows = (size_t)dims->num_seqs * dims->num_q_heads;
  const size_t o_bytes = (size_t)num_splits * rows * dims->head_dim * sizeof(float);
  p.part_o = need ? static_cast<float*>(workspace) : nullptr;
  p.part_lse = need ? reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                               ((o_bytes + 255) & ~(size_t)255))
                    : nullptr;
  p.num_seqs = dims->num_seqs;
  p.hq = dims->num_q_heads;
  p.hkv = dims->num_kv_heads;
  p.group = dims->num_q_heads / dims->num_kv_heads;
  p.num_blocks = dims->num_blocks;
  p.max_blocks = dims->max_blocks_per_seq;
  p.rel_len = dims->rel_len;
  p.window = window;
  p.num_splits = num_splits;
  p.chunk_tiles = decode_chunk_tiles(dims, window, num_splits);
  p.pid_cap = 2 * p.chunk_tiles + 16;
  p.max_seq_len = dims->max_seq_len;
  p.scale = scale;
  // A visible distance exceeds R - 1 only when the window (or, on global
  // layers, the longest context) is longer than the bias.
  const int64_t max_vis_d = window > 0 ? (int64_t)window - 1 : (int64_t)dims->max_seq_len - 1;
  p.clamp = max_vis_d > dims->rel_len - 1 ? 1 : 0;
  const size_t esz = dtype_size(dims->dtype);
  // As many adjacent KV heads per workgroup as divide Hkv and fit in LDS
  // (bf16); a single head per workgroup otherwise.
  p.heads_per_wg = 1;
  if (dims->dtype == 0) {
    for (int nh = kDecodeMaxHeadsPerWG; nh > 1; nh /= 2) {
      p.heads_per_wg = nh;
      if (dims->num_kv_heads % nh == 0 &&
          decode_lds_bytes(p, dims->dtype, dims->head_dim) <= 160 * 1024)
        break;
      p.heads_per_wg = 1;
    }
  }
  if (decode_lds_bytes(p, dims->dtype, dims->head_dim) > 160 * 1024)
    return INKLING_ERR_UNSUPPORTED;
  // 32-bit buffer offsets: one page, and the bias rows of one KV head.
  if ((int64_t)16 * dims->num_kv_heads * dims->head_dim * (int64_t)esz >= (1LL << 31) ||
      (int64_t)p.group * dims->rel_len * (int64_t)esz >= (1LL << 30))
    return INKLING_ERR_UNSUPPORTED;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = launch_decode(p, dims->dtype, dims->head_dim, s);
  if (e != hipSuccess) return INKLING_ERR_LAUNCH;
  if (num_splits > 1) {
    CombineParams c{};
    c.part_o = p.part_o;
    c.part_lse = p.part_lse;
    c.out = out;
    c.rows = (int32_t)rows;
    c.num_splits = num_splits;
    e = launch_combine(c, dims->dtype, dims->head_dim, s);
    if (e != hipSuccess) return INKLING_ERR_LAUNCH;
  }
  return INKLING_OK;
}

}  // namespace

extern "C" {

inkling_status_t inkling_rel_attn_prefill(const void* q, const void* k_cache, const void* v_cache,
                                          const int32_t* block_table, const int32_t* seq_lens,
                                          const int32_t* cu_q_lens, const void* rel_logits,
                                          int32_t window, float scale, void* out,
                                          const inkling_rel_attn_dims_t* dims, void* stream) {
  return prefill_impl(q, nullptr, nullptr, k_cache, v_cache, block_table, seq_lens, cu_q_lens,
                      rel_logits, window, scale, out, dims, stream);
}

inkling_status_t inkling_rel_attn_prefill_append(
    const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
    const int32_t* block_table, const int32_t* seq_lens, const int32_t* cu_q_lens,
    const void* rel_logits, int32_t window, float scale, void* out,
    const inkling_rel_attn_dims_t* dims, void* stream) {
  if (dims != nullptr && dims->total_q > 0 && (k_new == nullptr || v_new == nullptr))
    return INKLING_ERR_INVALID_ARGUMENT;
  return prefill_impl(q, k_new, v_new, k_cache, v_cache, block_table, seq_lens, cu_q_lens,
                      rel_logits, window, scale, out, dims, stream);
}

inkling_status_t inkling_rel_attn_decode(const void* q, const void* k_cache, const void* v_cache,
                                         const int32_t* block_table, const int32_t* seq_lens,
                                         const void* rel_logits, int32_t window, float scale,
                                         int32_t num_splits, void* workspace,
                                         size_t workspace_bytes, void* out,
                                         const inkling_rel_attn_dims_t* dims, void* stream) {
  return decode_impl(q, nullptr, nullptr, k_cache, v_cache, block_table, seq_lens, rel_logits,
                     window, scale, num_splits, workspace, workspace_bytes, out, dims, stream);
}

inkling_status_t inkling_rel_attn_decode_noalloc(const void* q, const void* k_cache,
                                                 const void* v_cache, const int32_t* block_table,
                                                 const int32_t* seq_lens, const void* rel_logits,
                                                 int32_t window, float scale, int32_t num_splits,
                                                 void* out, const inkling_rel_attn_dims_t* dims,
                                                 void* stream) {
  // Host-side checks first: nothing here touches a device before the
  // arguments are known to be valid and the split workspace to fit.
  inkling_status_t st = check_dims(dims);
  if (st != INKLING_OK) return st;
  if (num_splits < 0 || num_splits > kMaxSplits) return INKLING_ERR_INVALID_ARGUMENT;
  if (dims->num_seqs == 0) return INKLING_OK;
  if (num_splits > 0 && workspace_for(dims, num_splits) > decode_scratch_bytes())
    return INKLING_ERR_WORKSPACE_TOO_SMALL;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return INKLING_ERR_NO_DEVICE;
  }
  const int32_t splits = num_splits == 0 ? splits_for(dims, window, device_cus(dev)) : num_splits;
  if (workspace_for(dims, splits) > decode_scratch_bytes()) return INKLING_ERR_WORKSPACE_TOO_SMALL;
  void* ws = nullptr;
  if (decode_scratch(dev, &ws) != hipSuccess || ws == nullptr) {
    (void)hipGetLastError();
    return INKLING_ERR_LAUNCH;
  }
  return decode_impl(q, nullptr, nullptr, k_cache, v_cache, block_table, seq_lens, rel_logits,
                     window, scale, splits, ws, decode_scratch_bytes(), out, dims, stream);
}

inkling_status_t inkling_rel_attn_decode_append(
    const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
    const int32_t* block_table, const int32_t* seq_lens, const void* rel_logits, int32_t window,
    float scale, int32_t num_splits, void* workspace, size_t workspace_bytes, void* out,
    const inkling_rel_attn_dims_t* dims, void* stream) {
  if (dims != nullptr && dims->num_seqs > 0 && (k_new == nullptr || v_new == nullptr))
    return INKLING_ERR_INVALID_ARGUMENT;
  return decode_impl(q, k_new, v_new, k_cache, v_cache, block_table, seq_lens, rel_logits,
                     window, scale, num_splits, workspace, workspace_bytes, out, dims, stream);
}

}  // extern "C"
