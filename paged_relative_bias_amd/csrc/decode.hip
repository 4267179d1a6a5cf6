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
// workgroup.  The G query heads of the KV head are the MFMA columns (G <=
// 16).  Each wave walks 32-key tiles of the split round-robin and keeps its
// own online-softmax state; the four states are merged through LDS at the
// end.  Per tile:
//   K rows are read straight into MFMA A-operand registers (16-byte loads,
//   16 keys x 64 bytes per instruction);
//   S^T[key][head] = K . Q^T with 16x16x32 bf16 MFMA;
//   x = scale * S + bias | -inf, bias read per lane from its row;
//   V rows go to a wave-private LDS buffer and come back as the V^T
//   operand; O^T[d][head] += V^T . P^T with P kept in registers.
// With one split the workgroup writes the output directly; otherwise it
// writes its normalised partial and log-sum-exp, and combine_kernel merges
// them in a fixed order (no atomics, bit-reproducible).
#include <type_traits>

#include "device.hpp"
#include "launch.hpp"

namespace ira {
namespace {

template <typename T, int D>
struct Decode {
  static constexpr bool kBF16 = sizeof(T) == 2;
  static constexpr int NK = kDecodeKeys;            // keys per wave tile
  static constexpr int VSP = D + 4;                 // V row pitch in LDS
  static constexpr int QSTEPS = kBF16 ? D / 32 : D / 4;
  using Op = typename std::conditional<kBF16, bf16x8, float>::type;
  static constexpr size_t lds_bytes() {
    const size_t vbuf = (size_t)kDecodeWaves * NK * VSP * sizeof(T);
    const size_t merge = (size_t)kDecodeWaves * 16 * (D + 2) * sizeof(float);
    return vbuf > merge ? vbuf : merge;
  }
};

template <typename T, int D>
__global__ void __launch_bounds__(256)
decode_kernel(const DecodeParams P) {
  using C = Decode<T, D>;
  constexpr int NK = C::NK, VSP = C::VSP;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

  const T* __restrict__ qg = static_cast<const T*>(P.q);
  const T* __restrict__ kg = static_cast<const T*>(P.k);
  const T* __restrict__ vg = static_cast<const T*>(P.v);
  const T* __restrict__ rg = static_cast<const T*>(P.rel);

  const int split = blockIdx.x, b = blockIdx.y, g = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, u4 = lane >> 4;
  const int G = P.group, R = P.rel_len, W = P.window;
  const int64_t hq = P.hq;
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

  typename C::Op qop[C::QSTEPS];
  {
    const T* src = qg + ((int64_t)b * hq + h) * D;
    if constexpr (C::kBF16) {
#pragma unroll
      for (int s = 0; s < C::QSTEPS; ++s)
        qop[s] = cval ? *reinterpret_cast<const bf16x8*>(src + 32 * s + 8 * u4) : bf16x8{};
    } else {
#pragma unroll
      for (int s = 0; s < C::QSTEPS; ++s) qop[s] = cval ? src[4 * s + u4] : 0.f;
    }
  }
  const T* relrow = rg + ((int64_t)b * hq + h) * R;
  const int64_t bt_row = (int64_t)b * P.max_blocks;

  f32x4 acc[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) acc[dt] = f32x4{};
  float m_run = kNegInf, l_run = 0.f;
  T* Vs = reinterpret_cast<T*>(smem) + wave * NK * VSP;

  for (int kt = s_lo + NK * wave; kt < s_hi; kt += NK * kDecodeWaves) {
    // Gather K (as A operand) and V for keys kt + 16*blk + col.
    typename C::Op ka[2][C::QSTEPS];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const int j = kt + 16 * blk + col;
      const bool ok = j >= v_lo && j < s_hi;
      int64_t off = 0;
      if (ok) {
        const int page = iclamp(P.block_table[bt_row + (j >> 4)], 0, P.num_blocks - 1);
        off = (((int64_t)page * 16 + (j & 15)) * P.hkv + g) * D;
      }
      if constexpr (C::kBF16) {
#pragma unroll
        for (int s = 0; s < C::QSTEPS; ++s) {
          const int d0 = 32 * s + 8 * u4;
          ka[blk][s] = ok ? *reinterpret_cast<const bf16x8*>(kg + off + d0) : bf16x8{};
          const bf16x8 vv = ok ? *reinterpret_cast<const bf16x8*>(vg + off + d0) : bf16x8{};
          T* dst = Vs + (16 * blk + col) * VSP + d0;
          *reinterpret_cast<bf16x4*>(dst) = bf16x4{vv[0], vv[1], vv[2], vv[3]};
          *reinterpret_cast<bf16x4*>(dst + 4) = bf16x4{vv[4], vv[5], vv[6], vv[7]};
        }
      } else {
#pragma unroll
        for (int s = 0; s < C::QSTEPS; ++s) {
          const int d0 = 4 * s + u4;
          ka[blk][s] = ok ? kg[off + d0] : 0.f;
          Vs[(16 * blk + col) * VSP + d0] = ok ? vg[off + d0] : 0.f;
        }
      }
    }
    // S^T blocks: lane holds head `col`, keys kt + 16*blk + 4*u4 + i.
    f32x4 s[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      s[blk] = f32x4{};
#pragma unroll
      for (int st = 0; st < C::QSTEPS; ++st) s[blk] = mfma16(ka[blk][st], qop[st], s[blk]);
    }
    float x[8];
    float mx = kNegInf;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int j = kt + 16 * (i >> 2) + 4 * u4 + (i & 3);
      const int d = pq - j;
      const bool vis = cval && j >= v_lo && j < s_hi && (W <= 0 || d < W);
      const float bias = vis ? to_f32(relrow[imin(d, R - 1)]) : 0.f;
      x[i] = vis ? fmaf(s[i >> 2][i & 3], P.scale, bias) : kNegInf;
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
    // V writes above must land before other lanes read them back.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if constexpr (C::kBF16) {
      bf16x8 pb;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const bf16 r = from_f32<bf16>(fast_exp2(fmaf(x[i], kLog2e, -mb)));
        pb[i] = r;
        lsum += to_f32(r);
      }
      // A operand V^T: row d = 16*dt + col, contraction slots (u4, e) ->
      // keys 4*u4 + e (e < 4) and 16 + 4*u4 + e - 4 (e >= 4), matching pb.
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) {
        const T* vc = Vs + 16 * dt + col;
        bf16x8 a;
#pragma unroll
        for (int e = 0; e < 8; ++e) a[e] = vc[(16 * (e >> 2) + 4 * u4 + (e & 3)) * VSP];
        acc[dt] = mfma16(a, pb, acc[dt]);
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
    // Reads of Vs finish before the next tile overwrites it.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
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
  const dim3 grid(p.num_splits, p.num_seqs, p.hkv);
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
