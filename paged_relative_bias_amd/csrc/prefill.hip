// Varlen prefill: relative-bias attention over a paged KV cache on gfx950.
//
// Operation (TensorRT-LLM Inkling page, section "Architecture"): logits are
// scale * q.k plus a learned bias indexed by (query token, head, distance),
// masked to the causal prefix or to a sliding window, softmax over keys,
// weighted sum of values.  The paged prefill kernel of the same page
// (section "Implementation") is the prior art; this is a gfx950 design.
//
// Work decomposition.  One workgroup per (block of `bq` query tokens,
// sequence b, KV head g); the 1-D grid is remapped so that each of the 8
// XCDs receives a contiguous run of work, i.e. consecutive query blocks of
// one (b, g), whose key ranges overlap, share that XCD's L2.  The MFMA
// columns of a workgroup are its (query head in group, token) pairs,
// token-major (column c: head g*G + c % G, token t0 + c / G); each wave
// owns 32 columns, i.e. about 32 / G consecutive tokens of every head, so
// its visible key range is narrow (and the rows of a short sequence, such
// as a decode row, fill the first waves only).
//
// Key tiles of 32 keys sweep the union of the block's visible ranges,
// double-buffered in LDS:
//   * K rows and V rows are gathered through the block table: each wave
//     loads 8 keys of the tile (one page) through a buffer descriptor that
//     ends at the block's last key (later keys, and tiles past the last,
//     read zero without traffic); the page ids of the block's range sit in
//     an LDS table; they go through registers into rows with a 16-byte (K)
//     or 32-byte (V) pad (bf16 with head_dim 128 runs the specialised
//     kernel of prefill_bf16.hip instead);
//   * every wave copies the bias runs of its 32 rows for the tile: for
//     (token, head) the tile needs one contiguous run of the distance axis,
//     taken from an aligned window of sb entries with 16-byte loads;
//   * the next tile's loads are issued (into the other LDS stage, or into
//     registers written to it after the current tile is computed) before
//     the current tile is computed; the barriers order LDS only, so the
//     loads stay in flight across them.
// Per wave and tile:
//   S^T[key][col] = K . Q^T       32x32x16 bf16 MFMA (32x32x2 f32 for fp32)
//   x = scale * S + bias          mask by select only on boundary tiles
//   online softmax per column     two lanes per column (l, l ^ 32); the
//                                 reference max is the column's max in its
//                                 first tile with a visible key, raised
//                                 (with the column's accumulators rescaled
//                                 in registers) only on a tile where a
//                                 logit exceeds it by more than kOver
//   O^T[d][col] += V^T . P^T      V^T operand from ds_read_tr16_b64, P^T
//                                 from registers as two bf16 terms (hi =
//                                 RNE(P), lo = RNE(P - hi)), two MFMAs;
//                                 row sums of P in fp32.
// Issue order within a tile (bf16): bias runs and V^T operands are read
// from LDS first, so that their latency runs under the QK MFMAs and the
// softmax; the hi-term PV MFMAs go out before the lo terms and the row sum
// are computed, which then run under them.
#include <mutex>
#include <type_traits>

#include "device.hpp"
#include "launch.hpp"

namespace ira {
namespace {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));

// Largest logit excess over the reference (natural units) for which P =
// exp(x - m_ref) and the running sums stay far from fp32 / bf16 overflow.
constexpr float kOver = 40.f;

template <typename T, int D>
struct Prefill {
  static constexpr bool kBF16 = sizeof(T) == 2;
  static constexpr int N = kPrefillKeys;                 // keys per tile
  static constexpr int VEC = 16 / (int)sizeof(T);        // elements per 16 B
  static constexpr int CPR = D / VEC;                    // chunks per K/V row
  static constexpr int KP = D + VEC;                     // K row pitch
  static constexpr int VP = kBF16 ? D + 16 : D + 4;      // V row pitch
  static constexpr int QSTEPS = kBF16 ? D / 16 : D / 2;  // MFMA k-steps over D
  static constexpr int KPI = 64 / CPR;                   // keys per wave load
  static constexpr int KW = N / kPrefillWaves;           // keys each wave loads
  static constexpr int LPT = KW / KPI;                   // its loads per tensor
  static constexpr int KV_PER = 2 * LPT;                 // K then V
  static constexpr int SBC_MAX = (N + VEC) / VEC;        // bias chunks per row
  static constexpr int BIAS_PER = (32 * SBC_MAX + 63) / 64;
  using QOp = typename std::conditional<kBF16, bf16x8, float>::type;
  static constexpr size_t stage_bytes() { return (size_t)(N * KP + N * VP) * sizeof(T); }
};

template <typename T>
__device__ __forceinline__ void store4(T* dst, float a, float b, float c, float d) {
  if constexpr (sizeof(T) == 2) {
    bf16x4 v = {from_f32<bf16>(a), from_f32<bf16>(b), from_f32<bf16>(c), from_f32<bf16>(d)};
    *reinterpret_cast<bf16x4*>(dst) = v;
  } else {
    *reinterpret_cast<f32x4*>(dst) = f32x4{a, b, c, d};
  }
}

// Workgroup barrier that orders LDS only: in-flight global loads of the
// issuing waves are not waited for.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// APPEND: the new tokens' K/V rows come from P.k_new / P.v_new and are
// stored into the cache (a separate instantiation, so the plain kernel's
// loads stay free of control flow).
template <typename T, int D, bool APPEND>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
prefill_kernel(const PrefillParams P) {
  using C = Prefill<T, D>;
  constexpr int N = C::N, VEC = C::VEC, CPR = C::CPR, KP = C::KP, VP = C::VP, KPI = C::KPI;
  constexpr uint32_t SZ = sizeof(T);
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  constexpr int nw = kPrefillWaves;
  const int G = P.group, bq = P.bq, R = P.rel_len, SB = P.sb, W = P.window;
  // A key at distance d is visible when 0 <= d < W (any d >= 0 without a
  // window): one unsigned compare against wlim.
  const uint32_t wlim = W > 0 ? (uint32_t)W : 0x80000000u;
  const int64_t hq = P.hq;

  // XCD-aware work index: workgroup id x runs on XCD x % 8; give each XCD
  // a contiguous range of work (query block fastest, heaviest first).
  const int total = P.nqb * P.num_seqs * P.hkv;
  const int per_xcd = (total + 7) >> 3;
  const int w = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
  if (w >= total) return;
  const int qb = P.nqb - 1 - w % P.nqb;
  const int bg = w / P.nqb;
  const int b = bg % P.num_seqs, g = bg / P.num_seqs;

  // Sequence metadata, clamped so that no read leaves the arguments.
  const int q0 = iclamp(P.cu_q_lens[b], 0, P.total_q);
  const int q1 = iclamp(P.cu_q_lens[b + 1], q0, P.total_q);
  const int L = iclamp(P.seq_lens[b], 0, P.max_blocks * 16);
  const int n = imin(q1 - q0, L);
  const int t0 = qb * bq;
  if (t0 >= n) return;
  const int tend = imin(t0 + bq, n);
  const int pbase = L - n;                                  // position of token 0
  const int jb = W > 0 ? imax(0, pbase + t0 - W + 1) : 0;   // block's first key
  const int je = pbase + tend;                              // one past last key

  // This lane's column (query head, token).
  const int col = lane & 31, u = lane >> 5;
  const int wc = wave * 32 + col;
  const int hh = wc % G;
  const int tc = t0 + wc / G;
  const bool cval = hh < G && tc < tend;
  const int h = g * G + (hh < G ? hh : 0);
  const int pc = pbase + tc;
  // The wave's token range and its visible key range.
  const int c_lo = wave * 32, c_hi = imin(c_lo + 31, G * bq - 1);
  const int wt_lo = t0 + c_lo / G;
  const int wt_hi = imin(t0 + c_hi / G + 1, tend);   // exclusive
  const bool wact = c_lo < G * bq && wt_lo < tend;
  const int wjb = W > 0 ? imax(0, pbase + wt_lo - W + 1) : 0;
  const int wje = pbase + wt_hi;

  // LDS: two stages of (K tile, V tile), per-wave bias runs (two stages),
  // then the page-id table.
  auto stage = [&](int st) { return reinterpret_cast<T*>(smem + st * C::stage_bytes()); };
  unsigned char* bias_lds = smem + 2 * C::stage_bytes();
  const int sbp = P.sb_pitch;
  int* pid_lds = reinterpret_cast<int*>(bias_lds + (size_t)nw * 2 * 32 * sbp);

  // Page ids of keys [jb, je).
  const int pg_lo = jb >> 4;
  const int npg = imin(((je - 1) >> 4) - pg_lo + 1, P.pid_cap);
  {
    const int seq_pages = (L + 15) >> 4;
    const __amdgpu_buffer_rsrc_t bt_rsrc =
        make_rsrc(P.block_table + (int64_t)b * P.max_blocks, (uint32_t)seq_pages * 4u);
    for (int i = tid; i < npg; i += blockDim.x)
      pid_lds[i] = iclamp((int)bload32(bt_rsrc, (uint32_t)(pg_lo + i) * 4u), 0, P.num_blocks - 1);
  }

  typename C::QOp qop[C::QSTEPS];
  {
    const T* qg = static_cast<const T*>(P.q);
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
  }

  const uint32_t slot_bytes = (uint32_t)P.hkv * D * SZ;
  const uint32_t page_bytes = 16u * slot_bytes;
  const uint32_t head_bytes = (uint32_t)g * D * SZ;
  const char* kg = static_cast<const char*>(P.k);
  const char* vg = static_cast<const char*>(P.v);
  // Append: the new tokens' rows (keys pbase .. je - 1) are read from
  // k_new / v_new, never from the cache, and each workgroup stores its own
  // tokens' rows into the cache, so no workgroup waits for another's store.
  constexpr bool app = APPEND;
  const uint64_t kn = reinterpret_cast<uint64_t>(P.k_new);
  const uint64_t vn = reinterpret_cast<uint64_t>(P.v_new);
  // Bias rows of tokens [t0, tend), all heads: row (t, h') at
  // ((t - t0) * Hq + h') * R.
  const T* rel_base = static_cast<const T*>(P.rel) + (int64_t)(q0 + t0) * hq * R;
  const uint32_t rel_bytes = (uint32_t)(tend - t0) * (uint32_t)hq * (uint32_t)R * SZ;
  const int sbc = SB / VEC;  // bias chunks per row

  // ---- loads of one tile into registers ---------------------------------
  struct Regs {
    uint4 kv[C::KV_PER];
    uint4 b[C::BIAS_PER];
  };
  // Lane constants of the loads (independent of the tile).  Wave w loads
  // keys KW*w .. KW*w + KW - 1 of the tile (one page: tiles start at
  // multiples of 16); its load i of K (and of V) covers keys KW*w + KPI*i +
  // lane / CPR, 16-byte chunk lane % CPR.
  uint32_t kv_lane[C::LPT];
#pragma unroll
  for (int i = 0; i < C::LPT; ++i) {
    const int row = C::KW * wave + KPI * i + lane / CPR;
    kv_lane[i] = (uint32_t)(row & 15) * slot_bytes + head_bytes + (uint32_t)(lane % CPR) * 16u;
  }
  // Bias load i: row r = c / sbc (token rt, head rh), chunk c % sbc.
  uint32_t b_row[C::BIAS_PER];   // row offset | 0x80000000 if the row is unused
  // First entry of the row's window at kt = 0: floor_to(p - (N - 1), VEC);
  // tiles start at multiples of 16, so the window of tile kt starts kt
  // entries lower (before the clamp to [0, R - SB]).
  int b_fb[C::BIAS_PER];
#pragma unroll
  for (int i = 0; i < C::BIAS_PER; ++i) {
    const int c = i * 64 + lane;
    const int r = c / sbc, part = c - r * sbc;
    const int rc = wave * 32 + r;
    const int rh = rc % G, rt = t0 + rc / G;
    const bool ok = r < 32 && rh < G && rt < tend;
    b_row[i] = ((uint32_t)((rt - t0) * hq + g * G + rh) * (uint32_t)R + (uint32_t)(part * VEC)) * SZ |
               (ok ? 0u : kOOB);
    b_fb[i] = floor_to(pbase + rt - (N - 1), VEC);
  }
  // Loads of tile kt.  The K/V descriptors of the wave's page end at key
  // je (keys past it, and whole tiles past the last, read zero without
  // traffic); keys before jb are real cache rows.  Rows the wave does not
  // stage read as kOOB.  No control flow around any load.
  auto issue = [&](Regs& rg, int kt, int st_to) {
    {
      const int key0 = kt + C::KW * wave;                 // wave-uniform
      const int pgi = imin((key0 >> 4) - pg_lo, P.pid_cap - 1);   // >= 0
      const uint64_t page = (uint32_t)__builtin_amdgcn_readfirstlane(pid_lds[pgi]);
      // Keys of the page up to je (0 past the last tile), as a scalar.
      const int nk = __builtin_amdgcn_readfirstlane(je - (key0 & ~15));
      const uint32_t nrec = sgpr_u32((uint32_t)(nk <= 0 ? 0 : (nk >= 16 ? 16 : nk)) * slot_bytes);
      // With an append, slot s of this page is new token (key0 & ~15) + s -
      // pbase: the new rows are addressed like a page whose base sits
      // (key0 & ~15) - pbase rows from k_new's token q0 (only slots of new
      // tokens are ever read through it).
      const uint64_t new_off =
          (uint64_t)((int64_t)(q0 + (key0 & ~15) - pbase) * (int64_t)slot_bytes);
      const bool all_new = app && key0 >= pbase;         // wave-uniform
      const uint64_t kb =
          sgpr_u64(all_new ? kn + new_off : reinterpret_cast<uint64_t>(kg) + page * page_bytes);
      const uint64_t vb =
          sgpr_u64(all_new ? vn + new_off : reinterpret_cast<uint64_t>(vg) + page * page_bytes);
      const __amdgpu_buffer_rsrc_t rk = make_rsrc(reinterpret_cast<const void*>(kb), nrec);
      const __amdgpu_buffer_rsrc_t rv = make_rsrc(reinterpret_cast<const void*>(vb), nrec);
#pragma unroll
      for (int i = 0; i < C::LPT; ++i) {
        rg.kv[i] = bload128(rk, kv_lane[i]);
        rg.kv[C::LPT + i] = bload128(rv, kv_lane[i]);
      }

    }
    // Tiles the wave does not compute read no bias (an empty descriptor).
    const bool wtile = wact && kt < wje && kt + N > wjb;  // wave-uniform
    const __amdgpu_buffer_rsrc_t rr = make_rsrc(rel_base, sgpr_u32(wtile ? rel_bytes : 0u));
#pragma unroll
    for (int i = 0; i < C::BIAS_PER; ++i) {
      // Distances [p - kt - N + 1, p - kt] clamped to R - 1 lie in the
      // aligned window [base, base + SB).
      const int base = iclamp(b_fb[i] - kt, 0, R - SB);
      rg.b[i] = bload128(rr, b_row[i] + (uint32_t)base * SZ);
    }
  };
  // Tile kt's loads into LDS stage st.
  auto commit = [&](const Regs& rg, int st, int kt) {
    T* Ks = stage(st);
    T* Vs = Ks + N * KP;
#pragma unroll
    for (int i = 0; i < C::LPT; ++i) {
      const int key = C::KW * wave + KPI * i + lane / CPR;
      const int chunk = (lane % CPR) * VEC;
      *reinterpret_cast<uint4*>(Ks + key * KP + chunk) = rg.kv[i];
      *reinterpret_cast<uint4*>(Vs + key * VP + chunk) = rg.kv[C::LPT + i];
    }
    if constexpr (APPEND) {
      const int key0 = kt + C::KW * wave;                 // wave-uniform
      if (key0 < pbase && key0 + C::KW > pbase) {         // rare
        // The wave's keys cross the first new token: the rows staged above
        // for its new keys came from the cache; replace them with the new
        // rows.
        const uint64_t new_off =
            (uint64_t)((int64_t)(q0 + (key0 & ~15) - pbase) * (int64_t)slot_bytes);
        const uint32_t nrec = sgpr_u32((uint32_t)iclamp(je - (key0 & ~15), 0, 16) * slot_bytes);
        const __amdgpu_buffer_rsrc_t nk =
            make_rsrc(reinterpret_cast<const void*>(sgpr_u64(kn + new_off)), nrec);
        const __amdgpu_buffer_rsrc_t nv =
            make_rsrc(reinterpret_cast<const void*>(sgpr_u64(vn + new_off)), nrec);
#pragma unroll
        for (int i = 0; i < C::LPT; ++i) {
          const int key = C::KW * wave + KPI * i + lane / CPR;
          const int chunk = (lane % CPR) * VEC;
          const bool isnew = kt + key >= pbase;
          const uint4 a = bload128(nk, isnew ? kv_lane[i] : kOOB);
          const uint4 c = bload128(nv, isnew ? kv_lane[i] : kOOB);
          if (isnew) {
            *reinterpret_cast<uint4*>(Ks + key * KP + chunk) = a;
            *reinterpret_cast<uint4*>(Vs + key * VP + chunk) = c;
          }
        }
      }
    }
    unsigned char* Bw = bias_lds + (size_t)(wave * 2 + st) * 32 * sbp;
#pragma unroll
    for (int i = 0; i < C::BIAS_PER; ++i) {
      const int c = i * 64 + lane;
      const int r = c / sbc, part = c - r * sbc;
      if (r < 32) {
        uint32_t* dst = reinterpret_cast<uint32_t*>(Bw + r * sbp + part * 16);
        dst[0] = rg.b[i].x;
        dst[1] = rg.b[i].y;
        dst[2] = rg.b[i].z;
        dst[3] = rg.b[i].w;
      }
    }
  };

  f32x16 acc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) acc[dt] = f32x16{};
  // Softmax reference of the column (the two lanes of a column agree on it):
  // the max of its logits in its first tile with a visible key.  Later
  // logits may exceed it; P = exp(x - m_ref) stays far from overflow while
  // they exceed it by at most kOver.  On a tile where a logit exceeds it by
  // more, the column's reference becomes that tile's column max and its
  // accumulators and row sum are multiplied by exp(old - new), in registers
  // and only on that tile.
  // Lane constants of compute(): the column's bias window start at kt = 0
  // (tiles start at multiples of 16) and its lane's distance base.
  const int fpc = floor_to(pc - (N - 1), VEC);
  const int pcu = pc - 4 * u;
  float m_ref = kNegInf;
  float l_run = 0.f;

  // ---- compute one tile from LDS stage st --------------------------------
  auto compute = [&](int kt, int st) {
    if (!(wact && kt < wje && kt + N > wjb)) return;      // wave-uniform
    const T* Ks = stage(st);
    const T* Vs = Ks + N * KP;
    const T* brow = reinterpret_cast<const T*>(bias_lds + (size_t)(wave * 2 + st) * 32 * sbp +
                                               col * sbp);
    const int base_c = iclamp(fpc - kt, 0, R - SB);
    const int D0 = pcu - kt;
    // Bias runs of the fast path, read before the QK product so that their
    // LDS latency overlaps it (in-bounds for every lane; unused on the
    // general path).
    uint2 brun[4];
    if constexpr (C::kBF16) {
      const T* bb = brow + imin(D0 - base_c - 27, SB - 28);
#pragma unroll
      for (int k = 0; k < 4; ++k) __builtin_memcpy(&brun[k], bb + 24 - 8 * k, 8);
    }
    // V^T operands of this tile (bf16).  The plain kernel reads them here,
    // so that their LDS latency runs under the QK product and the softmax
    // arithmetic; the append instance reads them just before the PV product
    // (reading them early makes it spill).
    bf16x8 va[D / 32][2];
    auto read_vt = [&]() {
      if constexpr (C::kBF16) {
        // V^T operand for 16 keys ks*16 + slots (u, e): keys 16ks + 4u + e
        // (e < 4) and 16ks + 8 + 4u + e - 4 (e >= 4), matching ph/pl[ks].  The
        // 16-lane groups of a transposed read cover d0..d0+15: lane j points
        // at key (4u + j/4), columns d0 + 4*(j%4) .. +3.  All of them are read
        // before the first PV MFMA, as both P terms use them.
        const int jj = lane & 15;
        const int dgrp = (lane >> 4) & 1;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          const T* vb = Vs + (4 * u + (jj >> 2)) * VP + 32 * dt + 16 * dgrp + 4 * (jj & 3);
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) i16x4*)(vb + (16 * ks) * VP));
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) i16x4*)(vb + (16 * ks + 8) * VP));
            const i16x8 a16 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            va[dt][ks] = __builtin_bit_cast(bf16x8, a16);
          }
        }
      }
    };
    if constexpr (C::kBF16 && !APPEND) read_vt();
    f32x16 s = f32x16{};
    if constexpr (C::kBF16) {
      const bf16* krow = Ks + col * KP + 8 * u;
#pragma unroll
      for (int st2 = 0; st2 < C::QSTEPS; ++st2)
        s = mfma32(*reinterpret_cast<const bf16x8*>(krow + 16 * st2), qop[st2], s);
    } else {
      const float* krow = Ks + col * KP + u;
#pragma unroll
      for (int st2 = 0; st2 < C::QSTEPS; ++st2) s = mfma32(krow[2 * st2], qop[st2], s);
    }
    // x = scale * S + bias (natural-log units); lane holds keys
    // kt + 8*(i/4) + 4*u + i%4, i.e. distances d_i = pc - kt - 4u - c_i with
    // c_i = 8*(i/4) + i%4.
    float x[16];
    float mx = kNegInf;
    // Element i sits at distance d_i = D0 - c_i, D0 = pc - kt - 4u,
    // c_i = 8*(i/4) + i%4 (compile-time), and its bias at offset d_i -
    // base_c of the staged run: one base per lane plus immediate offsets.
    // Tiles with no distance at the clamp read the run directly and mask by
    // select (only on tiles that cross the window or causal boundary);
    // tiles that reach the clamp take the general path.
    const bool unclamped = (wje - 1) - kt <= R - 1;       // wave-uniform
    const bool full = (W <= 0 || (wje - 1) - kt < W) && (pbase + wt_lo) - (kt + N - 1) >= 0;
    if (unclamped) {
      // Entries start .. start + 27 of the staged run; for real columns
      // start + 27 <= SB - 1 on these tiles, and the bound keeps padding
      // columns' reads inside the staging area as well.
      if constexpr (C::kBF16) {
        // Run k holds entries 24 - 8k .. 27 - 8k; x[4k + j] takes entry
        // 27 - 8k - j.
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          x[4 * k + 0] = fmaf(s[4 * k + 0], P.scale, __builtin_bit_cast(float, brun[k].y & 0xffff0000u));
          x[4 * k + 1] = fmaf(s[4 * k + 1], P.scale, __builtin_bit_cast(float, brun[k].y << 16));
          x[4 * k + 2] = fmaf(s[4 * k + 2], P.scale, __builtin_bit_cast(float, brun[k].x & 0xffff0000u));
          x[4 * k + 3] = fmaf(s[4 * k + 3], P.scale, __builtin_bit_cast(float, brun[k].x << 16));
        }
      } else {
        const T* bb = brow + imin(D0 - base_c - 27, SB - 28);
#pragma unroll
        for (int i = 0; i < 16; ++i)
          x[i] = fmaf(s[i], P.scale, to_f32(bb[27 - (8 * (i >> 2) + (i & 3))]));
      }
      if (!full) {                                        // wave-uniform
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int d = D0 - (8 * (i >> 2) + (i & 3));
          const bool vis = (uint32_t)d < wlim;            // 0 <= d < window
          x[i] = vis ? x[i] : kNegInf;
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int d = D0 - (8 * (i >> 2) + (i & 3));
        // di is always inside the staged run, so the read is unconditional.
        const int di = iclamp(imin(d, R - 1) - base_c, 0, SB - 1);
        const float bv = to_f32(brow[di]);
        const bool vis = (uint32_t)d < wlim;
        x[i] = vis ? fmaf(s[i], P.scale, bv) : kNegInf;
      }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, x[i]);
    // A column's first tile with a visible key sets its reference (from
    // -inf: the factor is 0 and the accumulators are still 0); a logit more
    // than kOver above the reference raises it.  A column without a visible
    // key keeps -inf (then P = 0).  Padding columns (no such head or token)
    // may see arbitrary staged values and never take the branch.
    if (__builtin_amdgcn_ballot_w64(cval && mx > m_ref + kOver)) {   // wave-uniform, rare
      const float mc = fmaxf(mx, xor_lane(mx, 32));
      if (cval && mc > m_ref + kOver) {
        const float alpha = fast_exp2((m_ref - mc) * kLog2e);
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) acc[dt] *= alpha;
        l_run *= alpha;
        m_ref = mc;
      }
    }
    const float mb = m_ref == kNegInf ? 0.f : m_ref * kLog2e;
    if constexpr (C::kBF16) {
      // P enters the PV product as two bf16 terms, hi = RNE(P) and lo =
      // RNE(P - hi), whose sum is P to 2^-17 relative; a single bf16 P would
      // move an output by up to 2^-9 of the spread of V.
      // Exponentials and the hi terms first; the lo terms and the row sum
      // are computed while the hi-term MFMAs run.
      float pv[16];
      uint32_t hw[8];
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        pv[i] = fast_exp2(fmaf(x[i], kLog2e, -mb));
        pv[i + 1] = fast_exp2(fmaf(x[i + 1], kLog2e, -mb));
        hw[i >> 1] = bf16x2_hi(pv[i], pv[i + 1]);
      }
      bf16x8 ph[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        ph[ks] = __builtin_bit_cast(bf16x8, u32x4{hw[4 * ks], hw[4 * ks + 1], hw[4 * ks + 2],
                                                  hw[4 * ks + 3]});
      if constexpr (APPEND) read_vt();
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) acc[dt] = mfma32(va[dt][ks], ph[ks], acc[dt]);
      uint32_t lw[8];
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        lw[i >> 1] = bf16x2_lo(pv[i], pv[i + 1], hw[i >> 1]);
        l_run += pv[i];
        l_run += pv[i + 1];
      }
      bf16x8 pl[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        pl[ks] = __builtin_bit_cast(bf16x8, u32x4{lw[4 * ks], lw[4 * ks + 1], lw[4 * ks + 2],
                                                  lw[4 * ks + 3]});
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) acc[dt] = mfma32(va[dt][ks], pl[ks], acc[dt]);
    } else {
      float pf[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        pf[i] = fast_exp2(fmaf(x[i], kLog2e, -mb));
        l_run += pf[i];
      }
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        const float* vrow = Vs + 4 * u * VP + 32 * dt + col;
#pragma unroll
        for (int i = 0; i < 16; ++i)
          acc[dt] = mfma32(vrow[(8 * (i >> 2) + (i & 3)) * VP], pf[i], acc[dt]);
      }
    }
  };

  // ---- software pipeline over key tiles ----------------------------------
  // One register buffer: at the top of each step tile kt sits in an LDS
  // stage and tile kt+N is issued into the buffer; it lands while tile kt
  // is computed and goes to the other stage after.  (A second buffer, for
  // a tile more in flight, measured no faster and costs 28 VGPRs.)  Loads
  // past the last tile read nothing, so no load sits under control flow.
  if (app) {                                             // uniform
    // Store this workgroup's tokens' new K/V rows of head g into the cache.
    lds_barrier();                                       // page ids ready
    const int chunks = (tend - t0) * 2 * CPR;
    for (int c = tid; c < chunks; c += blockDim.x) {
      const int t = t0 + c / (2 * CPR), r = c % (2 * CPR);
      const bool isv = r >= CPR;
      const int ch = isv ? r - CPR : r;
      const int key = pbase + t;
      // The table holds npg pages from pg_lo; with valid metadata every new
      // key's page is among them (clipped tables only follow from lengths
      // above max_seq_len, whose result is unspecified: skip the store).
      const int pi = (key >> 4) - pg_lo;
      if (pi >= npg) continue;
      const uint64_t page = (uint32_t)pid_lds[pi];
      const uint64_t dst = page * page_bytes + (uint64_t)(key & 15) * slot_bytes + head_bytes +
                           (uint64_t)ch * 16u;
      const uint64_t src = ((uint64_t)(q0 + t) * P.hkv + g) * D * SZ + (uint64_t)ch * 16u;
      const uint4 v = *reinterpret_cast<const uint4*>((isv ? vn : kn) + src);
      *reinterpret_cast<uint4*>(reinterpret_cast<char*>(const_cast<void*>(isv ? P.v : P.k)) + dst) = v;
    }
  }
  Regs ra;
  lds_barrier();                                         // page ids ready
  int kt = jb & ~15;
  issue(ra, kt, 0);
  commit(ra, 0, kt);
  if (kt < jb) {                                         // workgroup-uniform
    // The first page holds keys before the block's first visible key: their
    // P is 0 for every column, but a non-finite V row would still turn 0 * V
    // into NaN in the PV product, so their V rows are zeroed.
    __builtin_amdgcn_s_waitcnt(0);
    lds_barrier();
    T* Vs = stage(0) + N * KP;
    for (int c = tid; c < (jb - kt) * CPR; c += blockDim.x)
      *reinterpret_cast<uint4*>(Vs + (c / CPR) * VP + (c % CPR) * VEC) = make_uint4(0u, 0u, 0u, 0u);
  }
  lds_barrier();
  while (true) {
    issue(ra, kt + N, 1);
    compute(kt, 0);
    if (kt + N >= je) break;                             // workgroup-uniform
    commit(ra, 1, kt + N);
    lds_barrier();
    kt += N;
    issue(ra, kt + N, 0);
    compute(kt, 1);
    if (kt + N >= je) break;
    commit(ra, 0, kt + N);
    lds_barrier();
    kt += N;
  }
  // Prefetches past the last tile may be outstanding: drain them before the
  // wave ends.
  __builtin_amdgcn_s_waitcnt(0);

  if (!wact) return;
  const float lt = l_run + xor_lane(l_run, 32);
  if (!cval) return;
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  T* dst = static_cast<T*>(P.out) + ((int64_t)(q0 + tc) * hq + h) * D;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4)
      store4(dst + 32 * dt + 8 * q4 + 4 * u, acc[dt][4 * q4] * inv, acc[dt][4 * q4 + 1] * inv,
             acc[dt][4 * q4 + 2] * inv, acc[dt][4 * q4 + 3] * inv);
}

template <typename T, int D>
size_t lds_bytes_t(int waves, int sb_pitch, int pid_cap) {
  return 2 * Prefill<T, D>::stage_bytes() + (size_t)waves * 2 * 32 * sb_pitch +
         (size_t)pid_cap * 4;
}

template <typename T, int D, bool APPEND>
hipError_t launch_a(const PrefillParams& p, hipStream_t stream) {
  const size_t lds = lds_bytes_t<T, D>(kPrefillWaves, p.sb_pitch, p.pid_cap);
  // Raise the kernel's dynamic LDS limit once per process (thread-safe).
  static std::once_flag once;
  static hipError_t attr = hipSuccess;
  std::call_once(once, [] {
    attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&prefill_kernel<T, D, APPEND>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  });
  if (attr != hipSuccess) return attr;
  const int64_t total = (int64_t)p.nqb * p.num_seqs * p.hkv;
  const int64_t grid = ((total + 7) / 8) * 8;
  prefill_kernel<T, D, APPEND><<<dim3((unsigned)grid), dim3(kPrefillWaves * 64), lds, stream>>>(p);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_t(const PrefillParams& p, hipStream_t stream) {
  return p.k_new != nullptr ? launch_a<T, D, true>(p, stream) : launch_a<T, D, false>(p, stream);
}

}  // namespace

size_t prefill_lds_bytes(int dtype, int head_dim, int waves, int sb_pitch, int pid_cap) {
  if (dtype == 0)
    return head_dim == 64 ? lds_bytes_t<bf16, 64>(waves, sb_pitch, pid_cap)
                          : lds_bytes_t<bf16, 128>(waves, sb_pitch, pid_cap);
  return head_dim == 64 ? lds_bytes_t<float, 64>(waves, sb_pitch, pid_cap)
                        : lds_bytes_t<float, 128>(waves, sb_pitch, pid_cap);
}

hipError_t launch_prefill(const PrefillParams& p, int dtype, int head_dim, hipStream_t stream) {
  // bf16 with head_dim 128 runs prefill_bf16_kernel (launch_prefill_bf16).
  if (dtype == 0) return head_dim == 64 ? launch_t<bf16, 64>(p, stream) : hipErrorInvalidValue;
  return head_dim == 64 ? launch_t<float, 64>(p, stream) : launch_t<float, 128>(p, stream);
}

}  // namespace ira
