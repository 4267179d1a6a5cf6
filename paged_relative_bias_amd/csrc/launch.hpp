// Kernel parameter blocks and launchers shared by the host ABI (abi.cpp) and
// the kernel translation units.  Internal to the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ira {

// Keys per prefill key tile and per decode wave tile.
constexpr int kPrefillKeys = 32;
// Prefill workgroups have 4 waves: 128 MFMA columns = G heads x
// floor(128 / G) query tokens.
constexpr int kPrefillWaves = 4;
constexpr int kDecodeKeys = 32;
// Decode waves per compute unit the split heuristic aims for (one per SIMD).
// A decode workgroup holds up to kDecodeMaxHeadsPerWG KV heads, one wave
// each, which load their tiles together.
constexpr int kDecodeWavesPerCU = 4;
constexpr int kDecodeMaxHeadsPerWG = 2;
constexpr int kMaxSplits = 128;
constexpr int kMaxGroup = 16;

struct PrefillParams {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const int32_t* cu_q_lens;
  const void* rel;
  void* out;
  const void* k_new;  // [total_q, Hkv, D] rows of the new tokens (keys L - n ..
  const void* v_new;  //   L - 1), stored into the cache and used (null: none)
  int32_t hq, hkv, group;
  int32_t num_blocks, max_blocks, rel_len, window, total_q;
  int32_t bq;         // query tokens per workgroup
  int32_t sb;         // bias entries staged per row and key tile
  int32_t sb_pitch;   // bytes between staged bias rows
  int32_t nqb;        // query blocks per sequence (ceil(max_q_len / bq))
  int32_t num_seqs;
  int32_t pid_cap;    // entries of the per-workgroup page-id table
  float scale;
};

struct DecodeParams {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const void* rel;
  void* out;          // final output (num_splits == 1)
  const void* k_new;  // [B, Hkv, D] rows stored at key L_b - 1 and used as it
  const void* v_new;  //   (both null: no append)
  float* part_o;      // [splits, B, Hq, D] normalised partial outputs
  float* part_lse;    // [splits, B, Hq]
  int32_t num_seqs, hq, hkv, group;
  int32_t num_blocks, max_blocks, rel_len, window, num_splits;
  int32_t chunk_tiles;  // 32-key tiles per split
  int32_t pid_cap;      // entries of the per-workgroup page-id table (>= 2 * chunk_tiles + 16)
  int32_t heads_per_wg; // KV heads (one wave each) per workgroup: 2 or 1 (bf16 only above 1)
  int32_t max_seq_len;  // host bound on seq_lens
  int32_t clamp;        // 1: a visible distance may exceed rel_len - 1
  float scale;
};

struct CombineParams {
  const float* part_o;
  const float* part_lse;
  void* out;
  int32_t rows;       // B * Hq
  int32_t num_splits;
};

// dtype: 0 = bf16, 1 = fp32.  Return the launch's hipError_t.
hipError_t launch_prefill(const PrefillParams& p, int dtype, int head_dim, hipStream_t stream);
size_t prefill_lds_bytes(int dtype, int head_dim, int waves, int sb_pitch, int pid_cap);
// The bf16, head_dim 128 prefill without append (the serving shapes).
hipError_t launch_prefill_bf16(const PrefillParams& p, hipStream_t stream);
size_t prefill_bf16_lds_bytes();
hipError_t launch_decode(const DecodeParams& p, int dtype, int head_dim,
                         hipStream_t stream);
size_t decode_lds_bytes(const DecodeParams& p, int dtype, int head_dim);
hipError_t launch_combine(const CombineParams& p, int dtype, int head_dim,
                          hipStream_t stream);
// The library's own split workspace on `device` (a file-scope device array):
// its size, and its device address, looked up once per device.
size_t decode_scratch_bytes();
hipError_t decode_scratch(int device, void** ptr);

}  // namespace ira
