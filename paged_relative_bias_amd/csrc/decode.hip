// Single-token decode with split-KV and a log-sum-exp merge, on gfx950.
//
// Operation: the relative-bias attention of the TensorRT-LLM Inkling page
// (section "Architecture") for one new token per sequence at position
// L_b - 1.  The split of each sequence's keys into parts, each producing a
// normalised partial output plus its log-sum-exp, followed by a merge, is
// the split-KV decode the vLLM page describes (section "Changes": up to 128
// splits, with a helper that picks the count).
//
// Work decomposition.  Grid (split, sequence, KV head); 4 waves per
// workgroup, each owning a contiguous run of 32-key tiles of the split.
// The G query heads of the KV head are the MFMA columns (G <= 16).
//
// The kernel is bound by HBM bandwidth, so the loop is built to keep loads
// in flight:
//   * each wave reads the page ids of its range once (one page per lane)
//     and takes them with readlane, so no tile waits on the block table;
//   * K, V and bias loads for tile t+1 are issued before tile t is
//     computed (two register buffers, loop unrolled by two);
//   * K is read straight into MFMA A-operand registers (16 keys x 64 bytes
//     per instruction); V is read as whole 256-byte rows and written to a
//     wave-private LDS tile whose 288-byte pitch keeps the transposed reads
//     free of bank conflicts.
// Per tile: S^T[key][head] = K . Q^T (16x16x32 bf16 MFMA); scale, bias,
// mask by select; online softmax with the column max shared across the
// four lanes of a column; O^T[d][head] += V^T . P^T where the V^T operand
// comes from ds_read_tr16_b64 (16 lanes each point at 4 consecutive d of
// one key; lane i receives that d-column for 4 keys) and P^T stays in
// registers.  The four waves' states are merged through LDS.  With one
// split the workgroup writes the output; otherwise it writes its
// normalised partial and log-sum-exp for combine_kernel, which merges the
// splits in a fixed order (no atomics, bit-reproducible).
#include <type_traits>

#include "device.hpp"
#include "launch.hpp"

namespace ira {
namespace {

typedef short i16x4 __attribute__((ext_vector_type(4)));

template <typename T, int D>
struct Decode {
  static constexpr bool kBF16 = sizeof(T) == 2;
  static constexpr int NK = kDecodeKeys;              // keys per wave tile
  static constexpr int CPR = D * (int)sizeof(T) / 16;  // 16-byte chunks per row
  static constexpr int VLOADS = NK * CPR / 64;        // V chunk loads per lane
  static constexpr int VSP = D + 16 / (int)sizeof(T) * 2;  // V row pitch (elements)
  static constexpr int KSTEPS = kBF16 ? D / 32 : D / 4;    // MFMA k-steps over D
  using KOp = typename std::conditional<kBF16, bf16x8, float>::type;
  static constexpr size_t lds_bytes() {
    const size_t vbuf = (size_t)kDecodeWaves * NK * VSP * sizeof(T);
    const size_t merge = (size_t)kDecodeWaves * 16 * (D + 2) * sizeof(float);
    return vbuf > merge ? vbuf : merge;
  }
};

// Registers holding one tile's K operands and raw bias values.
template <typename T, int D>
struct KBuf {
  using C = Decode<T, D>;
  typename C::KOp k[2][C::KSTEPS];
  uint32_t bias[8];
};

template <typename T>
__device__ __forceinline__ float raw_to_f32(uint32_t r) {
  if constexpr (sizeof(T) == 2) return __builtin_bit_cast(float, r << 16);
  else return __builtin_bit_cast(float, r);
}

template <typename T, int D>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
decode_kernel(const DecodeParams P) {
  using C = Decode<T, D>;
  constexpr int NK = C::NK, VSP = C::VSP, CPR = C::CPR, VEC = 16 / (int)sizeof(T);
  constexpr uint32_t SZ = sizeof(T);
  constexpr int kSegTiles = 128;                      // 256 pages per segment
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

  const T* __restrict__ qg = static_cast<const T*>(P.q);
  const char* kg = static_cast<const char*>(P.k);
  const char* vg = static_cast<const char*>(P.v);
  const T* __restrict__ rg = static_cast<const T*>(P.rel);

  // KV head fastest: the workgroups reading the Hkv interleaved rows of
  // the same pages run side by side.
  const int g = blockIdx.x, split = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, u4 = lane >> 4;
  const int G = P.group, R = P.rel_len, W = P.window;
  const int64_t hq = P.hq;
  const int hkv = P.hkv;
  const bool cval = col < G;
  const int h = g * G + (cval ? col : 0);

  const int L = iclamp(P.seq_lens[b], 0, P.max_blocks * 16);
  const int pq = L - 1;                               // query position
  const int k_lo = W > 0 ? imax(0, L - W) : 0;        // first visible key
  const int kb0 = k_lo & ~15;
  int chunk = (L - kb0 + P.num_splits - 1) / P.num_splits;
  chunk = (chunk + NK - 1) & ~(NK - 1);
  const int s_lo = kb0 + split * chunk;
  const int s_hi = imin(L, s_lo + chunk);
  const int v_lo = imax(s_lo, k_lo);                  // keys [v_lo, s_hi)
  const int ntiles = s_hi > s_lo ? (s_hi - s_lo + NK - 1) / NK : 0;
  const int tpw = (ntiles + kDecodeWaves - 1) / kDecodeWaves;
  const int t_begin = imin(ntiles, wave * tpw);
  const int t_end = imin(ntiles, t_begin + tpw);

  typename C::KOp qop[C::KSTEPS];
  {
    const T* src = qg + ((int64_t)b * hq + h) * D;
    if constexpr (C::kBF16) {
#pragma unroll
      for (int s = 0; s < C::KSTEPS; ++s)
        qop[s] = cval ? *reinterpret_cast<const bf16x8*>(src + 32 * s + 8 * u4) : bf16x8{};
    } else {
#pragma unroll
      for (int s = 0; s < C::KSTEPS; ++s) qop[s] = cval ? src[4 * s + u4] : 0.f;
    }
  }
  // Bias rows of the G heads of this KV head, R entries each.
  const __amdgpu_buffer_rsrc_t rel_rsrc =
      make_rsrc(rg + ((int64_t)b * hq + (int64_t)g * G) * R, (uint32_t)(G * R) * SZ);
  // Block-table row: entries of the sequence's pages only.
  const int seq_pages = (L + 15) >> 4;
  const __amdgpu_buffer_rsrc_t bt_rsrc =
      make_rsrc(P.block_table + (int64_t)b * P.max_blocks, (uint32_t)seq_pages * 4u);
  // One page holds 16 slots x Hkv heads x D; this head's row of slot s
  // starts at s * slot_bytes + head_bytes inside it.
  const uint32_t slot_bytes = (uint32_t)hkv * D * SZ;
  const uint32_t page_bytes = 16u * slot_bytes;
  const uint32_t head_bytes = (uint32_t)g * D * SZ;

  f32x4 acc[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) acc[dt] = f32x4{};
  float m_run = kNegInf, l_run = 0.f;
  // One LDS tile per wave, [key][VSP]; 16 lanes write one 256-byte row.
  // It is rewritten only after the previous tile's reads (same wave, LDS
  // ops in order), so the register copy in vreg is the only V prefetch.
  T* Vs = reinterpret_cast<T*>(smem) + wave * NK * VSP;

  for (int seg = t_begin; seg < t_end; seg += kSegTiles) {
    const int seg_end = imin(t_end, seg + kSegTiles);
    // Page ids of the segment: register r, lane i holds page pg_base+64r+i.
    const int pg_base = (s_lo >> 4) + 2 * seg;
    int pid[4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
      pid[r] = iclamp((int)bload32(bt_rsrc, (uint32_t)(pg_base + 64 * r + lane) * 4u), 0,
                      P.num_blocks - 1);
    auto page_rsrc = [&](const char* base, int seq_page) {
      const int p = iclamp(seq_page - pg_base, 0, 255);   // wave-uniform
      const int r = p >> 6;
      const int v = r == 0 ? pid[0] : r == 1 ? pid[1] : r == 2 ? pid[2] : pid[3];
      const int64_t page = __builtin_amdgcn_readlane(v, p & 63);
      return make_rsrc(base + page * page_bytes, page_bytes);
    };

    // K operands and raw bias of tile t; every lane loads unconditionally
    // (kOOB for keys outside the split and for t >= seg_end).
    auto load_k = [&](KBuf<T, D>& buf, int t) {
      const int kt = s_lo + t * NK;                   // multiple of 16
      const bool tile_ok = t < seg_end;
      const __amdgpu_buffer_rsrc_t r0 = page_rsrc(kg, kt >> 4);
      const __amdgpu_buffer_rsrc_t r1 = page_rsrc(kg, (kt >> 4) + 1);
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        const int j = kt + 16 * blk + col;
        const bool ok = tile_ok && j >= v_lo && j < s_hi;
        const uint32_t off = ok ? (uint32_t)(j & 15) * slot_bytes + head_bytes : kOOB;
        if constexpr (C::kBF16) {
#pragma unroll
          for (int st = 0; st < C::KSTEPS; ++st)
            buf.k[blk][st] = __builtin_bit_cast(
                bf16x8, bload128(blk ? r1 : r0, off + (uint32_t)(32 * st + 8 * u4) * SZ));
        } else {
#pragma unroll
          for (int st = 0; st < C::KSTEPS; ++st)
            buf.k[blk][st] = __builtin_bit_cast(
                float, bload32(blk ? r1 : r0, off + (uint32_t)(4 * st + u4) * SZ));
        }
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int j = kt + 16 * (i >> 2) + 4 * u4 + (i & 3);
        const bool vis = tile_ok && cval && j >= v_lo && j < s_hi;
        const uint32_t off = vis ? (uint32_t)(col * R + imin(pq - j, R - 1)) * SZ : kOOB;
        buf.bias[i] = C::kBF16 ? bload16(rel_rsrc, off) : bload32(rel_rsrc, off);
      }
    };

    // V rows of tile t: load i covers keys (i*64)/CPR .. +64/CPR, all in
    // page block (i*64/CPR) >> 4 of the tile.
    uint4 vreg[C::VLOADS];
    auto load_v = [&](int t) {
      const int kt = s_lo + t * NK;
      const bool tile_ok = t < seg_end;
      const __amdgpu_buffer_rsrc_t r0 = page_rsrc(vg, kt >> 4);
      const __amdgpu_buffer_rsrc_t r1 = page_rsrc(vg, (kt >> 4) + 1);
#pragma unroll
      for (int i = 0; i < C::VLOADS; ++i) {
        const int idx = i * 64 + lane;
        const int key = idx / CPR, ch = idx % CPR;
        const int j = kt + key;
        const bool ok = tile_ok && j >= v_lo && j < s_hi;
        const uint32_t off =
            ok ? (uint32_t)(j & 15) * slot_bytes + head_bytes + (uint32_t)ch * 16u : kOOB;
        vreg[i] = bload128(((i * 64 / CPR) >> 4) ? r1 : r0, off);
      }
    };
    auto store_v = [&]() {
#pragma unroll
      for (int i = 0; i < C::VLOADS; ++i) {
        const int idx = i * 64 + lane;
        const int key = idx / CPR, ch = idx % CPR;
        *reinterpret_cast<uint4*>(Vs + key * VSP + ch * VEC) = vreg[i];
      }
    };

    auto compute_tile = [&](const KBuf<T, D>& buf, int t) {
      const int kt = s_lo + t * NK;
      // S^T blocks: lane holds head `col`, keys kt + 16*blk + 4*u4 + i.
      f32x4 s[2];
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        s[blk] = f32x4{};
#pragma unroll
        for (int st = 0; st < C::KSTEPS; ++st) s[blk] = mfma16(buf.k[blk][st], qop[st], s[blk]);
      }
      float x[8];
      float mx = kNegInf;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int j = kt + 16 * (i >> 2) + 4 * u4 + (i & 3);
        const bool vis = cval && j >= v_lo && j < s_hi;
        x[i] = vis ? fmaf(s[i >> 2][i & 3], P.scale, raw_to_f32<T>(buf.bias[i])) : kNegInf;
        mx = fmaxf(mx, x[i]);
      }
      mx = fmaxf(mx, xor_lane(mx, 16));
      mx = fmaxf(mx, xor_lane(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      const float m_use = m_new == kNegInf ? 0.f : m_new;
      const float alpha = fast_exp2((m_run - m_use) * kLog2e);
      m_run = m_new;
      const float mb = m_use * kLog2e;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) acc[dt] *= alpha;
      float lsum = 0.f;
      if constexpr (C::kBF16) {
        bf16x8 pb;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const bf16 r = from_f32<bf16>(fast_exp2(fmaf(x[i], kLog2e, -mb)));
          pb[i] = r;
          lsum += to_f32(r);
        }
        // V^T operand: contraction slots (u4, e) hold keys 4*u4 + e (e < 4)
        // and 16 + 4*u4 + e - 4 (e >= 4), the keys of pb's slots.
        const int jj = lane & 15;
        const T* r0 = Vs + (4 * u4 + (jj >> 2)) * VSP + 4 * (jj & 3);
        const T* r1 = r0 + 16 * VSP;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4*)(r0 + 16 * dt));
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4*)(r1 + 16 * dt));
          typedef short i16x8 __attribute__((ext_vector_type(8)));
          const i16x8 a16 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          acc[dt] = mfma16(__builtin_bit_cast(bf16x8, a16), pb, acc[dt]);
        }
      } else {
        float pf[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          pf[i] = fast_exp2(fmaf(x[i], kLog2e, -mb));
          lsum += pf[i];
        }
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
          const T* vc = Vs + 16 * dt + col;
#pragma unroll
          for (int i = 0; i < 8; ++i)
            acc[dt] = mfma16(vc[(16 * (i >> 2) + 4 * u4 + (i & 3)) * VSP], pf[i], acc[dt]);
        }
      }
      l_run = l_run * alpha + lsum;
    };

    // Software pipeline, prefetch distance one tile for K, bias and V:
    //   iteration t: issue K/bias of t+1; compute t from its K registers and
    //   the LDS V tile; then store V of t+1 (loaded one iteration earlier)
    //   to the LDS tile and issue V of t+2.  Loads past the end are kOOB
    //   no-ops, so the loop body has no loads under control flow.  LDS ops of
    //   one wave run in order; the wave barriers only keep the compiler from
    //   moving LDS accesses across the hand-over.
    auto lds_handover = [&]() {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };
    KBuf<T, D> kA, kB;
    load_k(kA, seg);
    load_v(seg);
    store_v();
    load_v(seg + 1);
    lds_handover();
    for (int t = seg; t < seg_end; t += 2) {
      load_k(kB, t + 1);
      compute_tile(kA, t);
      if (t + 1 >= seg_end) break;
      lds_handover();
      store_v();
      load_v(t + 2);
      lds_handover();
      load_k(kA, t + 2);
      compute_tile(kB, t + 1);
      if (t + 2 >= seg_end) break;
      lds_handover();
      store_v();
      load_v(t + 3);
      lds_handover();
    }
    lds_handover();
  }

  // Merge the four waves' states.
  l_run += xor_lane(l_run, 16);
  l_run += xor_lane(l_run, 32);
  __syncthreads();
  float* ored = reinterpret_cast<float*>(smem);         // [wave][col][D]
  float* mred = ored + kDecodeWaves * 16 * D;           // [wave][col]
  float* lred = mred + kDecodeWaves * 16;
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      ored[(wave * 16 + col) * D + 16 * dt + 4 * u4 + i] = acc[dt][i];
  if (u4 == 0) {
    mred[wave * 16 + col] = m_run;
    lred[wave * 16 + col] = l_run;
  }
  __syncthreads();
  for (int idx = tid; idx < G * D; idx += blockDim.x) {
    const int c = idx / D, d = idx - c * D;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) M = fmaxf(M, mred[w * 16 + c]);
    float o = 0.f, lse = kNegInf;
    if (M != kNegInf) {
      float num = 0.f, den = 0.f;
#pragma unroll
      for (int w = 0; w < kDecodeWaves; ++w) {
        const float sc = expf(mred[w * 16 + c] - M);
        num += sc * ored[(w * 16 + c) * D + d];
        den += sc * lred[w * 16 + c];
      }
      o = num / den;
      lse = M + logf(den);
    }
    const int64_t row = (int64_t)b * hq + g * G + c;
    if (P.num_splits == 1) {
      static_cast<T*>(P.out)[row * D + d] = from_f32<T>(o);
    } else {
      const int64_t prow = (int64_t)split * P.num_seqs * hq + row;
      P.part_o[prow * D + d] = o;
      if (d == 0) P.part_lse[prow] = lse;
    }
  }
}

// One wave per (sequence, head) row; lane covers d = lane + 64 * k.
template <typename T, int D>
__global__ void __launch_bounds__(256)
combine_kernel(const CombineParams P) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= P.rows) return;
  const int lane = threadIdx.x & 63;
  constexpr int PER = D / 64;
  float M = kNegInf;
  for (int s = 0; s < P.num_splits; ++s)
    M = fmaxf(M, P.part_lse[(int64_t)s * P.rows + row]);
  float num[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) num[k] = 0.f;
  float den = 0.f;
  if (M != kNegInf) {
    for (int s = 0; s < P.num_splits; ++s) {
      const float l = P.part_lse[(int64_t)s * P.rows + row];
      if (l == kNegInf) continue;
      const float w = expf(l - M);
      den += w;
      const float* po = P.part_o + ((int64_t)s * P.rows + row) * D;
#pragma unroll
      for (int k = 0; k < PER; ++k) num[k] += w * po[lane + 64 * k];
    }
  }
  T* dst = static_cast<T*>(P.out) + (int64_t)row * D;
#pragma unroll
  for (int k = 0; k < PER; ++k)
    dst[lane + 64 * k] = from_f32<T>(den > 0.f ? num[k] / den : 0.f);
}

template <typename T, int D>
hipError_t launch_decode_t(const DecodeParams& p, hipStream_t stream) {
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&decode_kernel<T, D>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)Decode<T, D>::lds_bytes());
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const dim3 grid(p.hkv, p.num_splits, p.num_seqs);
  decode_kernel<T, D><<<grid, dim3(64 * kDecodeWaves), Decode<T, D>::lds_bytes(), stream>>>(p);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_combine_t(const CombineParams& p, hipStream_t stream) {
  combine_kernel<T, D><<<dim3((p.rows + 3) / 4), dim3(256), 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, int dtype, int head_dim,
                         hipStream_t stream) {
  if (dtype == 0)
    return head_dim == 64 ? launch_decode_t<bf16, 64>(p, stream)
                          : launch_decode_t<bf16, 128>(p, stream);
  return head_dim == 64 ? launch_decode_t<float, 64>(p, stream)
                        : launch_decode_t<float, 128>(p, stream);
}

hipError_t launch_combine(const CombineParams& p, int dtype, int head_dim,
                          hipStream_t stream) {
  if (dtype == 0)
    return head_dim == 64 ? launch_combine_t<bf16, 64>(p, stream)
                          : launch_combine_t<bf16, 128>(p, stream);
  return head_dim == 64 ? launch_combine_t<float, 64>(p, stream)
                        : launch_combine_t<float, 128>(p, stream);
}

}  // namespace ira
