// Varlen prefill: relative-bias attention over a paged KV cache on gfx950.
//
// Operation (TensorRT-LLM Inkling page, section "Architecture"): logits are
// scale * q.k plus a learned bias indexed by (query token, head, distance),
// masked to the causal prefix or to a sliding window, softmax over keys,
// weighted sum of values.  The paged prefill kernel of the same page
// (section "Implementation") is the prior art; this is a gfx950 design.
//
// Work decomposition.  One workgroup per (block of `bq` query tokens,
// sequence b, KV head g).  Its MFMA columns are the (query head in group,
// token) pairs, head-major: column c holds head g*G + c / bq and token
// t0 + c % bq.  Each wave owns 32 columns.  Key tiles of 64 keys sweep the
// union of the block's visible ranges; K/V rows are gathered through the
// block table into LDS (V transposed on the way in) and shared by all waves.
//
// Per wave and 32-key half tile:
//   S^T[key][col] = K . Q^T       32x32x16 bf16 MFMA (32x32x2 f32 for fp32)
//   x = scale * S + bias | -inf   bias row staged in LDS, masked by select
//   online softmax per column     two lanes per column (l, l ^ 32)
//   O^T[d][col] += V^T . P^T      P stays in registers as the B operand
// The column max/sum are exchanged with the partner lane only.  The bias
// for (token, head) over one key tile is a contiguous run of the
// distance axis; each wave copies the runs of its 32 rows with 16-byte
// loads, so every bias entry is read from memory about once.
#include <type_traits>

#include "device.hpp"
#include "launch.hpp"

namespace ira {
namespace {

template <typename T, int D>
struct Prefill {
  static constexpr bool kBF16 = sizeof(T) == 2;
  static constexpr int N = kPrefillKeys;              // keys per tile
  static constexpr int VEC = 16 / sizeof(T);          // elements per 16 B
  static constexpr int KP = D + VEC;                  // K row pitch (elements)
  static constexpr int VP = N + (kBF16 ? 4 : 1);      // V^T row pitch
  static constexpr int QSTEPS = kBF16 ? D / 16 : D / 2;
  using QOp = typename std::conditional<kBF16, bf16x8, float>::type;
  static constexpr size_t tile_bytes() {
    return (size_t)(N * KP + D * VP) * sizeof(T);
  }
};

template <typename T>
__device__ __forceinline__ void store4(T* dst, float a, float b, float c,
                                       float d) {
  if constexpr (sizeof(T) == 2) {
    bf16x4 v = {from_f32<bf16>(a), from_f32<bf16>(b), from_f32<bf16>(c),
                from_f32<bf16>(d)};
    *reinterpret_cast<bf16x4*>(dst) = v;
  } else {
    *reinterpret_cast<f32x4*>(dst) = f32x4{a, b, c, d};
  }
}

template <typename T, int D>
__global__ void __launch_bounds__(768)
prefill_kernel(const PrefillParams P) {
  using C = Prefill<T, D>;
  constexpr int N = C::N, VEC = C::VEC, KP = C::KP, VP = C::VP;
  constexpr int CPR = D / VEC;  // 16-byte chunks per K/V row
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  T* Ks = reinterpret_cast<T*>(smem);
  T* Vt = Ks + N * KP;
  unsigned char* Bs = smem + C::tile_bytes();

  const T* __restrict__ qg = static_cast<const T*>(P.q);
  const T* __restrict__ kg = static_cast<const T*>(P.k);
  const T* __restrict__ vg = static_cast<const T*>(P.v);
  const T* __restrict__ rg = static_cast<const T*>(P.rel);
  T* __restrict__ og = static_cast<T*>(P.out);

  const int b = blockIdx.y, g = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nthr = blockDim.x;
  const int G = P.group, bq = P.bq, R = P.rel_len, SB = P.sb, W = P.window;
  const int64_t hq = P.hq;

  // Sequence metadata, clamped so that no read leaves the arguments.
  const int q0 = iclamp(P.cu_q_lens[b], 0, P.total_q);
  const int q1 = iclamp(P.cu_q_lens[b + 1], q0, P.total_q);
  const int L = iclamp(P.seq_lens[b], 0, P.max_blocks * 16);
  const int n = imin(q1 - q0, L);
  // Later token blocks see more keys under full causal attention: start
  // them first.
  const int t0 = (gridDim.x - 1 - blockIdx.x) * bq;
  if (t0 >= n) return;
  const int tend = imin(t0 + bq, n);
  const int pbase = L - n;  // position of token 0 of this sequence
  const int jb = W > 0 ? imax(0, pbase + t0 - W + 1) : 0;  // block's first key
  const int je = pbase + tend;                              // one past last

  // This lane's column (query head, token).
  const int col = lane & 31, u = lane >> 5;
  const int wc = wave * 32 + col;
  const int hh = wc / bq;
  const int tc = t0 + wc % bq;
  const bool cval = hh < G && tc < tend;
  const int h = g * G + (hh < G ? hh : 0);
  const int pc = pbase + tc;
  // The wave's token range and visible key range.
  const int wt_lo = bq >= 32 ? t0 + (wave * 32) % bq : t0;
  const int wt_hi = imin(wt_lo + (bq >= 32 ? 32 : bq), tend);  // exclusive
  const bool wact = wt_lo < tend && (wave * 32) / bq < G;
  const int wjb = W > 0 ? imax(0, pbase + wt_lo - W + 1) : 0;
  const int wje = pbase + wt_hi;

  typename C::QOp qop[C::QSTEPS];
  if constexpr (C::kBF16) {
    const bf16* src = qg + ((int64_t)(q0 + tc) * hq + h) * D + 8 * u;
#pragma unroll
    for (int s = 0; s < C::QSTEPS; ++s)
      qop[s] = cval ? *reinterpret_cast<const bf16x8*>(src + 16 * s) : bf16x8{};
  } else {
    const float* src = qg + ((int64_t)(q0 + tc) * hq + h) * D + u;
#pragma unroll
    for (int s = 0; s < C::QSTEPS; ++s) qop[s] = cval ? src[2 * s] : 0.f;
  }

  f32x16 acc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) acc[dt] = f32x16{};
  float m_run = kNegInf, l_run = 0.f;

  const int64_t bt_row = (int64_t)b * P.max_blocks;
  const int sbp = P.sb_pitch;
  const int bias_cpr = SB / VEC;

  for (int kt = jb & ~15; kt < je; kt += N) {
    __syncthreads();  // previous tile fully consumed
    // K tile, row-major: consecutive lanes read consecutive 16-byte chunks.
    for (int c = tid; c < N * CPR; c += nthr) {
      const int kk = c / CPR, part = c - kk * CPR;
      const int j = kt + kk;
      uint4 val = make_uint4(0, 0, 0, 0);
      if (j >= jb && j < je) {
        const int page = iclamp(P.block_table[bt_row + (j >> 4)], 0, P.num_blocks - 1);
        val = *reinterpret_cast<const uint4*>(
            kg + (((int64_t)page * 16 + (j & 15)) * P.hkv + g) * D + part * VEC);
      }
      *reinterpret_cast<uint4*>(Ks + kk * KP + part * VEC) = val;
    }
    // V tile, transposed to V^T[d][key]: lanes take consecutive keys so each
    // LDS store writes one contiguous run of a V^T row.
    for (int c = tid; c < N * CPR; c += nthr) {
      const int kk = c % N, part = c / N;
      const int j = kt + kk;
      uint4 val = make_uint4(0, 0, 0, 0);
      if (j >= jb && j < je) {
        const int page = iclamp(P.block_table[bt_row + (j >> 4)], 0, P.num_blocks - 1);
        val = *reinterpret_cast<const uint4*>(
            vg + (((int64_t)page * 16 + (j & 15)) * P.hkv + g) * D + part * VEC);
      }
      const T* e = reinterpret_cast<const T*>(&val);
#pragma unroll
      for (int x = 0; x < VEC; ++x) Vt[(part * VEC + x) * VP + kk] = e[x];
    }
    // Bias runs of this wave's rows: distances [p - kt - N + 1, p - kt],
    // clamped to R - 1, taken from an aligned window of SB entries.
    const bool wtile = wact && kt < wje && kt + N > wjb;
    if (wtile) {
      unsigned char* Bw = Bs + wave * 32 * sbp;
      for (int c = lane; c < 32 * bias_cpr; c += 64) {
        const int r = c / bias_cpr, part = c - r * bias_cpr;
        const int rc = wave * 32 + r;
        const int rh = rc / bq, rt = t0 + rc % bq;
        uint4 val = make_uint4(0, 0, 0, 0);
        if (rh < G && rt < tend) {
          const int base = iclamp(floor_to(pbase + rt - kt - (N - 1), VEC), 0, R - SB);
          val = *reinterpret_cast<const uint4*>(
              rg + ((int64_t)(q0 + rt) * hq + g * G + rh) * R + base + part * VEC);
        }
        uint32_t* dst = reinterpret_cast<uint32_t*>(Bw + r * sbp + part * 16);
        dst[0] = val.x;
        dst[1] = val.y;
        dst[2] = val.z;
        dst[3] = val.w;
      }
    }
    __syncthreads();
    if (!wtile) continue;

    const T* brow = reinterpret_cast<const T*>(Bs + (wave * 32 + col) * sbp);
    const int base_c = iclamp(floor_to(pc - kt - (N - 1), VEC), 0, R - SB);
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      const int kb = kt + 32 * kh;
      if (kb >= wje || kb + 32 <= wjb) continue;  // wave-uniform
      // S^T for 32 keys x 32 columns.
      f32x16 s = f32x16{};
      if constexpr (C::kBF16) {
        const bf16* krow = Ks + (32 * kh + col) * KP + 8 * u;
#pragma unroll
        for (int st = 0; st < C::QSTEPS; ++st)
          s = mfma32(*reinterpret_cast<const bf16x8*>(krow + 16 * st), qop[st], s);
      } else {
        const float* krow = Ks + (32 * kh + col) * KP + u;
#pragma unroll
        for (int st = 0; st < C::QSTEPS; ++st) s = mfma32(krow[2 * st], qop[st], s);
      }
      // Scale, bias, mask; lane holds keys kb + 8*(i/4) + 4*u + i%4.
      float x[16];
      float mx = kNegInf;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int j = kb + 8 * (i >> 2) + 4 * u + (i & 3);
        const int d = pc - j;
        const bool vis = cval && d >= 0 && (W <= 0 || d < W);
        const int di = iclamp(imin(d, R - 1) - base_c, 0, SB - 1);
        const float bias = to_f32(brow[di]);
        x[i] = vis ? fmaf(s[i], P.scale, bias) : kNegInf;
        mx = fmaxf(mx, x[i]);
      }
      mx = fmaxf(mx, xor_lane(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      const float m_use = m_new == kNegInf ? 0.f : m_new;
      const float alpha = fast_exp2((m_run - m_use) * kLog2e);
      m_run = m_new;
      const float mb = m_use * kLog2e;
      float lsum = 0.f;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) acc[dt] *= alpha;
      if constexpr (C::kBF16) {
        // P rounded to bf16; the row sum uses the rounded values so the
        // weights applied to V are exactly normalised.
        bf16x8 pb[2];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const bf16 r = from_f32<bf16>(fast_exp2(fmaf(x[i], kLog2e, -mb)));
          pb[i >> 3][i & 7] = r;
          lsum += to_f32(r);
        }
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          const bf16* vrow = Vt + (32 * dt + col) * VP + 32 * kh + 4 * u;
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            const bf16x4 lo = *reinterpret_cast<const bf16x4*>(vrow + 16 * ks);
            const bf16x4 hi = *reinterpret_cast<const bf16x4*>(vrow + 16 * ks + 8);
            const bf16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            acc[dt] = mfma32(a, pb[ks], acc[dt]);
          }
        }
      } else {
        float pf[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          pf[i] = fast_exp2(fmaf(x[i], kLog2e, -mb));
          lsum += pf[i];
        }
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          const float* vrow = Vt + (32 * dt + col) * VP + 32 * kh + 4 * u;
#pragma unroll
          for (int i = 0; i < 16; ++i)
            acc[dt] = mfma32(vrow[8 * (i >> 2) + (i & 3)], pf[i], acc[dt]);
        }
      }
      l_run = l_run * alpha + lsum;
    }
  }

  if (!wact) return;
  const float lt = l_run + xor_lane(l_run, 32);
  if (!cval) return;
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  T* dst = og + ((int64_t)(q0 + tc) * hq + h) * D;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4)
      store4(dst + 32 * dt + 8 * q4 + 4 * u, acc[dt][4 * q4] * inv,
             acc[dt][4 * q4 + 1] * inv, acc[dt][4 * q4 + 2] * inv,
             acc[dt][4 * q4 + 3] * inv);
}

template <typename T, int D>
hipError_t launch_t(const PrefillParams& p, int num_seqs, int max_q_len,
                    hipStream_t stream) {
  const int waves = (p.group * p.bq + 31) / 32;
  const size_t lds = Prefill<T, D>::tile_bytes() + (size_t)waves * 32 * p.sb_pitch;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&prefill_kernel<T, D>),
        hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const dim3 grid((max_q_len + p.bq - 1) / p.bq, num_seqs, p.hkv);
  prefill_kernel<T, D><<<grid, dim3(waves * 64), lds, stream>>>(p);
  return hipGetLastError();
}

}  // namespace

size_t prefill_lds_bytes(int dtype, int head_dim, int waves, int sb_pitch) {
  size_t tile = 0;
  if (dtype == 0)
    tile = head_dim == 64 ? Prefill<bf16, 64>::tile_bytes() : Prefill<bf16, 128>::tile_bytes();
  else
    tile = head_dim == 64 ? Prefill<float, 64>::tile_bytes() : Prefill<float, 128>::tile_bytes();
  return tile + (size_t)waves * 32 * sb_pitch;
}

hipError_t launch_prefill(const PrefillParams& p, int dtype, int head_dim,
                          int num_seqs, int max_q_len, hipStream_t stream) {
  if (dtype == 0) {
    return head_dim == 64 ? launch_t<bf16, 64>(p, num_seqs, max_q_len, stream)
                          : launch_t<bf16, 128>(p, num_seqs, max_q_len, stream);
  }
  return head_dim == 64 ? launch_t<float, 64>(p, num_seqs, max_q_len, stream)
                        : launch_t<float, 128>(p, num_seqs, max_q_len, stream);
}

}  // namespace ira
