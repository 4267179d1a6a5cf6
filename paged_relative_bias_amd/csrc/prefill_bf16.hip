// Varlen prefill for bf16 with head_dim 128 (the serving shapes): relative-
// bias attention over a paged KV cache on gfx950.
//
// Operation (TensorRT-LLM Inkling page, section "Architecture"): logits are
// scale * q.k plus a learned bias indexed by (query token, head, distance),
// masked to the causal prefix or to a sliding window, softmax over keys,
// weighted sum of values.  The paged prefill kernel of the same page
// (section "Implementation") is the prior art; this is a gfx950 design.
//
// Work decomposition and columns are those of the generic prefill kernel:
// one workgroup per (block of bq query tokens, sequence b, KV head g) on an
// XCD-remapped 1-D grid, here sized from the batch's total query tokens
// rather than sequences x the longest; the 4 waves' 128 MFMA columns are
// (query head in group, token) pairs, token-major, 32 per wave.  Key tiles
// of 32 keys sweep the union of the block's visible ranges through two LDS
// stages; per wave
// and tile S^T = K . Q^T (32x32x16 bf16 MFMA), x = scale * S + bias, a
// softmax against a per-column reference (the column's max in its first
// tile with a visible key, raised, with the accumulators rescaled in
// registers, only on a tile where some logit exceeds it by more than
// kOver), and O^T += V^T . P^T with P as two bf16 terms (hi = RNE(P), lo =
// RNE(P - hi)).
//
// What differs from the generic kernel:
//   * Key order inside a tile.  LDS row r of a tile holds key
//     kperm(r) = 16 * ((r >> 2) & 1) + 4 * (r >> 3) + (r & 3).  The 32x32
//     MFMA puts S^T rows 8k + 4u + j (k < 4, j < 4) in lane half u, so with
//     this order lane half u holds keys 16u .. 16u + 15 of the tile, in
//     order: element i of a lane is key kt + 16u + i.  The contraction of
//     the PV product runs over LDS rows, so it needs no change; only the
//     rows' source slots move (wave w's load i fetches slots 4w .. 4w + 3 of
//     page i of the tile).
//   * Bias through LDS, two tiles ahead.  For every column the tile needs
//     one contiguous run of 32 distances of its bias row; the wave copies an
//     aligned 40-entry window of it (five 16-byte chunks, aligned to the row
//     so that none straddles a row or the buffer end) straight into its own
//     LDS region with 16-byte loads that have the LDS destination, into one
//     of three stages, two tiles ahead of the tile being computed.  A lane
//     then reads its 16 elements (distances D0 - 15 .. D0, D0 = p - kt - 16u)
//     as one 32-byte run at a lane-constant offset of its column's window.
//     Every load of the loop has the LDS destination and is invisible to the
//     compiler, so all waits are explicit counts.  Tiles where every visible
//     distance of the wave is at the clamp (d >= R - 1) use the column's
//     entry R - 1, read once; tiles whose visible distances straddle the
//     clamp read each element's clamped entry.
//   * K and V rows go from HBM straight into LDS (16-byte buffer loads with
//     the LDS destination) in the bank-conflict-free layout of the generic
//     kernel: K row r at byte r * 256 + 128 * (r >> 3), 16-byte chunk c at
//     c ^ (r & 7); V row r at byte r * 256, chunk c at c ^ (4 * (r & 3)).
//   * Fused append (a separate instance): pages whose keys are all new are
//     loaded from the new rows, the one page that straddles the first new
//     token is patched in LDS, and each workgroup stores its own tokens'
//     rows into the cache.
#include <mutex>

#include "device.hpp"
#include "launch.hpp"

namespace ira {
namespace {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));

// Largest logit excess over the reference (natural units) for which P =
// exp(x - m_ref) and the running sums stay far from fp32 / bf16 overflow.
constexpr float kOver = 40.f;

constexpr int kD = 128;                      // head_dim
constexpr int kN = kPrefillKeys;             // keys per tile (32)
constexpr uint32_t kKBytes = 8704;           // K region of a stage (32 rows + 3 x 128 B shift)
constexpr uint32_t kVBytes = 32 * 256;       // V region of a stage
constexpr uint32_t kStage = kKBytes + kVBytes;
// Bias windows: 40 entries (5 chunks of 16 bytes) per column and tile, 160
// chunks per wave, written by three 1 KB LDS-destination loads (the last
// one's upper half carries no column and writes zeros).
constexpr int kWinChunks = 5;
constexpr uint32_t kBiasWave = 3 * 1024;     // bytes per wave and bias stage
constexpr int kBiasStages = 3;
constexpr uint32_t kBiasOff = 2 * kStage;
constexpr uint32_t kLdsBytes = kBiasOff + (uint32_t)kBiasStages * kPrefillWaves * kBiasWave;

// Waits until at most N of this wave's vector-memory loads are in flight
// (the other counters are left alone).
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier that orders LDS only: in-flight global loads of the
// issuing waves are not waited for.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// fp32 value of the bf16 held in bits [15:0] of w.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }

// APPEND: the new tokens' K/V rows (keys pbase .. je - 1) come from
// P.k_new / P.v_new, never from the cache, and each workgroup stores its own
// tokens' rows into the cache, so no workgroup waits for another's store (a
// separate instantiation: the plain kernel's loads stay free of it).
template <bool APPEND>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
prefill_bf16_kernel(const PrefillParams P) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  constexpr uint32_t SZ = 2;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = P.group, bq = P.bq, R = P.rel_len, W = P.window;
  // A key at distance d is visible when 0 <= d < W (any d >= 0 without a
  // window): one unsigned compare against wlim.
  const uint32_t wlim = W > 0 ? (uint32_t)W : 0x80000000u;
  const int64_t hq = P.hq;

  // Work list.  Sequence b owns the block indices [S(b), S(b + 1)) with
  // S(b) = floor(cu_q_lens[b] / bq) + b: at least its ceil(n_b / bq) query
  // blocks and at most one more, NB = S(B) in all, so a batch of short rows
  // beside long chunks launches no workgroup per (row, unused block).  A
  // sequence's blocks run last (heaviest) first.  XCD-aware: workgroup id x
  // runs on XCD x % 8, and each XCD gets a contiguous range of the work, so
  // neighbouring query blocks of one (sequence, KV head) share its L2.
  const int Bn = P.num_seqs;
  const int NB = P.total_q / bq + Bn;
  const int total = NB * P.hkv;
  const int per_xcd = (total + 7) >> 3;
  const int w = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
  if (w >= total) return;
  const int j = w % NB, g = w / NB;
  // The sequence is the largest b with S(b) <= j (S increases with b).  Each
  // wave finds it on its own, from 64 candidates per round; metadata that
  // is not monotone still yields some b in [0, B).
  int b = 0, cq0 = 0, cq1 = 0, Lraw = 0;
  if (Bn <= 63) {
    // One round trip: lanes 0..B hold cu_q_lens, lanes 0..B-1 seq_lens.
    const int i = imin(lane, Bn);
    const int cq = iclamp(P.cu_q_lens[i], 0, P.total_q);
    const int sl = P.seq_lens[imin(lane, Bn - 1)];
    const uint64_t m = __builtin_amdgcn_ballot_w64(lane < Bn && cq / bq + lane <= j);
    b = imax(__builtin_popcountll(m) - 1, 0);
    cq0 = __builtin_amdgcn_readlane(cq, b);
    cq1 = __builtin_amdgcn_readlane(cq, b + 1);
    Lraw = __builtin_amdgcn_readlane(sl, b);
  } else {
    int span = Bn;                                       // b is in [b, b + span)
    while (span > 1) {                                   // wave-uniform
      const int step = (span + 63) / 64;
      const int idx = b + lane * step;
      const int S = lane * step < span ? iclamp(P.cu_q_lens[idx], 0, P.total_q) / bq + idx
                                       : 0x7fffffff;
      const uint64_t m = __builtin_amdgcn_ballot_w64(S <= j);
      b += imax(__builtin_popcountll(m) - 1, 0) * step;
      span = imin(step, Bn - b);
    }
    cq0 = iclamp(P.cu_q_lens[b], 0, P.total_q);
    cq1 = iclamp(P.cu_q_lens[b + 1], 0, P.total_q);
    Lraw = P.seq_lens[b];
  }
  const int qb = (cq1 / bq + b + 1) - 1 - j;             // S(b + 1) - 1 - j
  if (qb < 0) return;

  // Sequence metadata, clamped so that no read leaves the arguments.
  const int q0 = cq0;
  const int q1 = imax(cq1, q0);
  const int L = iclamp(Lraw, 0, P.max_blocks * 16);
  const int n = imin(q1 - q0, L);
  const int t0 = qb * bq;
  if (t0 >= n) return;
  const int tend = imin(t0 + bq, n);
  const int pbase = L - n;                                  // position of token 0
  const int jb = W > 0 ? imax(0, pbase + t0 - W + 1) : 0;   // block's first key
  const int je = pbase + tend;                              // one past last key

  // A block whose columns all fit one wave (G x tokens <= 32: single-token
  // rows of a mixed batch, a sequence's last few tokens) gives every wave
  // those columns and a quarter of the key tiles instead (tile i to wave
  // i mod 4); the waves' partial results are merged at the end.
  const bool ksplit = G * (tend - t0) <= 32;              // workgroup-uniform
  const int wsel = ksplit ? 0 : wave;
  // This lane's column (query head, token) and lane half.
  const int col = lane & 31, u = lane >> 5;
  const int wc = wsel * 32 + col;
  const int hh = wc % G;
  const int tc = t0 + wc / G;
  const bool cval = hh < G && tc < tend;
  const int h = g * G + (hh < G ? hh : 0);
  const int pc = pbase + tc;
  // The wave's token range and its visible key range.
  const int c_lo = wsel * 32, c_hi = imin(c_lo + 31, G * bq - 1);
  const int wt_lo = t0 + c_lo / G;
  const int wt_hi = imin(t0 + c_hi / G + 1, tend);   // exclusive
  const bool wact = c_lo < G * bq && wt_lo < tend;
  const int wjb = W > 0 ? imax(0, pbase + wt_lo - W + 1) : 0;
  const int wje = pbase + wt_hi;

  // LDS: two stages of (K tile, V tile) and three stages of the waves' bias
  // windows.  Page ids are read with scalar loads a tile ahead of their use,
  // so LDS does not grow with the context.  The sequence's block-table row
  // is read-only for the kernel's lifetime (constant address space).
  using const_i32 = const __attribute__((address_space(4))) int;
  const_i32* bt_row = (const_i32*)(P.block_table + (int64_t)b * P.max_blocks);
  const int last_page = imax(((L + 15) >> 4) - 1, 0);

  // Q^T operand (B of the QK MFMA), held for the whole kernel.
  bf16x8 qop[8];
  {
    const bf16* src = static_cast<const bf16*>(P.q) + ((int64_t)(q0 + tc) * hq + h) * kD + 8 * u;
#pragma unroll
    for (int s = 0; s < 8; ++s)
      qop[s] = cval ? *reinterpret_cast<const bf16x8*>(src + 16 * s) : bf16x8{};
  }

  const uint32_t slot_bytes = (uint32_t)P.hkv * kD * SZ;
  const uint32_t page_bytes = 16u * slot_bytes;
  const uint32_t head_bytes = (uint32_t)g * kD * SZ;
  const char* kg = static_cast<const char*>(P.k);
  const char* vg = static_cast<const char*>(P.v);
  const uint64_t kn = reinterpret_cast<uint64_t>(P.k_new);
  const uint64_t vn = reinterpret_cast<uint64_t>(P.v_new);
  // K/V loads.  Wave w's load i writes LDS rows 4 (2w + i) .. + 3 (one 1 KB
  // block, lane l at bytes 16 l .. 16 l + 15 after M0), which hold keys
  // 16 i + 4 w + l / 16: slot 4 w + l / 16 of page i of the tile.  Lane l
  // writes physical chunk l % 16 of its row, so it fetches the logical chunk
  // the layout puts there.
  uint32_t k_lane[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = 4 * (2 * wave + i) + (lane >> 4);
    k_lane[i] = (uint32_t)(4 * wave + (lane >> 4)) * slot_bytes + head_bytes +
                (uint32_t)((lane & 15) ^ (row & 7)) * 16u;
  }
  const uint32_t v_lane = (uint32_t)(4 * wave + (lane >> 4)) * slot_bytes + head_bytes +
                          (uint32_t)((lane & 15) ^ (4 * (lane >> 4))) * 16u;

  // Bias rows of tokens [t0, tend), all heads: row (t, h') at
  // ((t - t0) * Hq + h') * R entries after rel_base.
  const bf16* rel_base = static_cast<const bf16*>(P.rel) + (int64_t)(q0 + t0) * hq * R;
  const uint32_t rel_bytes = (uint32_t)(tend - t0) * (uint32_t)hq * (uint32_t)R * SZ;
  const __amdgpu_buffer_rsrc_t rel_rsrc = make_rsrc(rel_base, sgpr_u32(rel_bytes));
  const uint32_t row_off = (uint32_t)((tc - t0) * (int)hq + h) * (uint32_t)R * SZ;
  // Bias window of the tile at kt for a column at position p: entries
  // [w0, w0 + 40) of its row with w0 = floor_to(p - 31, 8) - kt (kt is a
  // multiple of 16), which holds distances p - kt - 31 .. p - kt.  LDS load
  // m of a wave writes chunks 64 m .. 64 m + 63 of its region: chunk c is
  // part c % 5 of column c / 5's window.  A chunk's entry lies on a multiple
  // of 8, and R is one: a chunk before its row's start or past its end holds
  // only masked distances (future keys, or distances >= R on a window tile),
  // so it reads the row's first or last chunk instead; reading it from the
  // neighbouring row would fetch that row's line a whole sweep before the
  // row's own column reaches it.  Chunks of padding columns, and of the last
  // load's upper half, read nothing.
  uint32_t b_dma[3];
  int b_pos[3];
#pragma unroll
  for (int m = 0; m < 3; ++m) {
    const int c = 64 * m + lane;
    const int bc = c / kWinChunks, part = c - bc * kWinChunks;
    const int rc = wsel * 32 + bc;
    const int rh = rc % G, rt = t0 + rc / G;
    const bool ok = bc < 32 && rh < G && rt < tend;
    const int w0 = floor_to(pbase + rt - (kN - 1), 8);
    b_dma[m] = ok ? (uint32_t)((rt - t0) * (int)hq + g * G + rh) * (uint32_t)R * SZ
                  : 0xf0000000u;      // past any bias buffer: reads zero
    b_pos[m] = w0 + 8 * part;
  }
  // The lane's 16 elements: entries D0 - 15 .. D0 of the window, i.e. 32
  // bytes from entry ((pc - 31) & 7) + 16 (1 - u) of its column's window.
  const uint32_t b_read = (uint32_t)col * (kWinChunks * 16) +
                          (uint32_t)(((pc - (kN - 1)) & 7) + 16 * (1 - u)) * SZ;
  // The column's entry R - 1, for tiles where every distance is clamped.
  const float bias_cl = cval ? bf16_lo(bload16(rel_rsrc, row_off + (uint32_t)(R - 1) * SZ)) : 0.f;
  // Drain the loads the compiler sees (Q, the clamp entry) before the loop:
  // its own waits count only those, so a later use of them would otherwise
  // wait for every LDS-destination load in flight.
  __builtin_amdgcn_s_waitcnt(0);

  // Tile kinds for this wave (all wave-uniform): the largest distance of the
  // wave's columns in the tile at kt is (wje - 1) - kt, the largest visible
  // one that or W - 1, the smallest (pbase + wt_lo) - (kt + 31).  A tile
  // whose visible distances all lie below R takes the runs; elements at
  // masked distances >= R read whatever follows their row (or zero past the
  // buffer) and are discarded.
  const int vis_cap = W > 0 ? W - 1 : 0x7fffffff;
  auto unclamped = [&](int kt) { return imin((wje - 1) - kt, vis_cap) <= R - 1; };
  auto all_clamped = [&](int kt) { return (pbase + wt_lo) - (kt + kN - 1) >= R - 1; };
  const int kt_first = jb & ~15;
  auto wave_tile = [&](int kt) {
    return wact && kt < wje && kt + kN > wjb && (!ksplit || ((kt - kt_first) >> 5) % kPrefillWaves == wave);
  };

  // K/V of the tile at kt into LDS stage st.  The descriptors of the tile's
  // two pages end at key je (keys past it, and whole tiles past the last,
  // read zero without traffic).  No control flow around any load.
  // The tile's two page ids.  Pages past the sequence's last read its last
  // page (such tiles' descriptors are empty), and every id is clamped into
  // the pool.
  auto page_ids = [&](int kt) {
    const int p0 = imin(kt >> 4, last_page), p1 = imin((kt >> 4) + 1, last_page);
    return make_int2(iclamp(bt_row[p0], 0, P.num_blocks - 1),
                     iclamp(bt_row[p1], 0, P.num_blocks - 1));
  };
  auto issue_kv = [&](int kt, int st, int2 pids) {
    const uint64_t page0 = (uint32_t)__builtin_amdgcn_readfirstlane(pids.x);
    const uint64_t page1 = (uint32_t)__builtin_amdgcn_readfirstlane(pids.y);
    const int nk = __builtin_amdgcn_readfirstlane(je - kt);
    const uint32_t n0 = sgpr_u32((uint32_t)(nk <= 0 ? 0 : (nk >= 16 ? 16 : nk)) * slot_bytes);
    const uint32_t n1 = sgpr_u32((uint32_t)(nk <= 16 ? 0 : (nk >= 32 ? 16 : nk - 16)) * slot_bytes);
    uint64_t kb0 = reinterpret_cast<uint64_t>(kg) + page0 * page_bytes;
    uint64_t kb1 = reinterpret_cast<uint64_t>(kg) + page1 * page_bytes;
    uint64_t vb0 = reinterpret_cast<uint64_t>(vg) + page0 * page_bytes;
    uint64_t vb1 = reinterpret_cast<uint64_t>(vg) + page1 * page_bytes;
    if constexpr (APPEND) {
      // A page whose keys are all new reads the new rows instead: slot s is
      // new token (page's first key + s - pbase), so the rows are addressed
      // like a page whose base sits that many rows after k_new's token q0.
      // (A page that straddles pbase reads the cache and is patched once it
      // has landed.)
      if (kt >= pbase) {                                 // wave-uniform
        const uint64_t off = (uint64_t)(q0 + kt - pbase) * slot_bytes;
        kb0 = kn + off;
        vb0 = vn + off;
      }
      if (kt + 16 >= pbase) {
        const uint64_t off = (uint64_t)(q0 + kt + 16 - pbase) * slot_bytes;
        kb1 = kn + off;
        vb1 = vn + off;
      }
    }
    const __amdgpu_buffer_rsrc_t rk0 = make_rsrc(reinterpret_cast<const void*>(sgpr_u64(kb0)), n0);
    const __amdgpu_buffer_rsrc_t rk1 = make_rsrc(reinterpret_cast<const void*>(sgpr_u64(kb1)), n1);
    const __amdgpu_buffer_rsrc_t rv0 = make_rsrc(reinterpret_cast<const void*>(sgpr_u64(vb0)), n0);
    const __amdgpu_buffer_rsrc_t rv1 = make_rsrc(reinterpret_cast<const void*>(sgpr_u64(vb1)), n1);
    // Block kb = 2 w + i: K at kb * 1024 + 128 * (kb >> 1), V at kKBytes +
    // kb * 1024.  The compiler does not see these loads; every wait for them
    // is explicit, and nothing else in the kernel uses M0.
    const uint32_t sl = sgpr_u32((uint32_t)st * kStage);
    const uint32_t kl0 = sgpr_u32(sl + (uint32_t)(2 * wave) * 1024u + 128u * (uint32_t)wave);
    const uint32_t kl1 = sgpr_u32(kl0 + 1024u);
    const uint32_t vl0 = sgpr_u32(sl + kKBytes + (uint32_t)(2 * wave) * 1024u);
    const uint32_t vl1 = sgpr_u32(vl0 + 1024u);
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :: "s"(kl0), "v"(k_lane[0]), "s"(rk0) : "memory", "m0");
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :: "s"(vl0), "v"(v_lane), "s"(rv0) : "memory", "m0");
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :: "s"(kl1), "v"(k_lane[1]), "s"(rk1) : "memory", "m0");
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :: "s"(vl1), "v"(v_lane), "s"(rv1) : "memory", "m0");
#pragma clang diagnostic pop
  };

  // Bias windows of the tile at kt into bias stage bs (tiles the wave
  // computes on the window path; for the others the loads read nothing and
  // write zeros).
  auto issue_bias = [&](int kt, int bs) {
    const bool win = wave_tile(kt) && unclamped(kt);       // wave-uniform
    const __amdgpu_buffer_rsrc_t rr = make_rsrc(rel_base, sgpr_u32(win ? rel_bytes : 0u));
    const uint32_t bl = sgpr_u32(kBiasOff + (uint32_t)(bs * kPrefillWaves + wave) * kBiasWave);
#pragma unroll
    for (int m = 0; m < 3; ++m) {
      const int pos = imin(imax(b_pos[m] - kt, 0), R - 8);
      const uint32_t off = b_dma[m] + (uint32_t)pos * SZ;
      const uint32_t ml = sgpr_u32(bl + 1024u * (uint32_t)m);
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
      asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                   :: "s"(ml), "v"(off), "s"(rr) : "memory", "m0");
#pragma clang diagnostic pop
    }
  };

  f32x16 acc[kD / 32];
#pragma unroll
  for (int dt = 0; dt < kD / 32; ++dt) acc[dt] = f32x16{};
  // Softmax reference of the column (the two lanes of a column agree on it):
  // the max of its logits in its first tile with a visible key.  Later
  // logits may exceed it; P = exp(x - m_ref) stays far from overflow while
  // they exceed it by at most kOver.  On a tile where a logit exceeds it by
  // more, the column's reference becomes that tile's column max and its
  // accumulators and row sum are multiplied by exp(old - new), in registers
  // and only on that tile; the common tile needs neither a cross-lane
  // exchange nor a rescale.
  float m_ref = kNegInf;
  float l_run = 0.f;

  // ---- compute one tile from LDS stage st ----------------------------------
  // `between` issues the loads of later tiles: it runs after this tile's
  // LDS reads are issued and before their first use, so that its scalar
  // work overlaps their latency.
  // pids are the next tile's page ids, loaded one step earlier.
  auto compute = [&](int kt, int st, int bs, int2 pids, auto&& between) {
    if (!wave_tile(kt)) {                                 // wave-uniform
      between(pids);
      return;
    }
    const bf16* Ks = reinterpret_cast<const bf16*>(smem + (size_t)st * kStage);
    const bf16* Vs = reinterpret_cast<const bf16*>(smem + (size_t)st * kStage + kKBytes);
    const int D0 = pc - kt - 16 * u;                       // distance of element 0
    // V^T operands of this tile, read first so that their LDS latency runs
    // under the QK product and the softmax.  Operand ks covers the S^T rows
    // of elements 8 ks .. 8 ks + 7: rows 4u + e (e < 4) and 8 + 4u + e - 4 of
    // the 16-row half ks.  The 16-lane groups of a transposed read cover
    // columns d0 .. d0 + 15: lane jj points at row 4u + jj / 4, columns
    // d0 + 4 (jj % 4) .. + 3.  Rows 4u + jj / 4 (+ 8, + 16) share r & 3 =
    // jj / 4, so d-block dt of the lane's columns starts 32 (dt ^ (jj / 4))
    // elements into the row.
    bf16x8 va[kD / 32][2];
    {
      const int jj = lane & 15;
      const int dgrp = (lane >> 4) & 1;
      const bf16* vbase = Vs + (4 * u + (jj >> 2)) * kD + 8 * (2 * dgrp + ((jj & 3) >> 1)) +
                          4 * (jj & 1);
#pragma unroll
      for (int dt = 0; dt < kD / 32; ++dt) {
        const bf16* vb = vbase + 32 * (dt ^ (jj >> 2));
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4*)(vb + (16 * ks) * kD));
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4*)(vb + (16 * ks + 8) * kD));
          const i16x8 a16 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          va[dt][ks] = __builtin_bit_cast(bf16x8, a16);
        }
      }
    }
    // K operands of S^T = K . Q^T.  Logical chunk 2 s + u of row col sits at
    // chunk (2 s + u) ^ (col & 7) = 2 ((s & 3) ^ y) + z + 8 (s >> 2).
    bf16x8 kop[8];
    {
      const int y = (col & 7) >> 1, z = u ^ (col & 1);
      const bf16* krow = Ks + col * kD + 64 * (col >> 3) + 8 * z;
#pragma unroll
      for (int s2 = 0; s2 < 8; ++s2)
        kop[s2] = *reinterpret_cast<const bf16x8*>(krow + 16 * ((s2 & 3) ^ y) + 64 * (s2 >> 2));
    }
    // The lane's bias run (window tiles): halfword m of its 32 bytes is
    // entry D0 - 15 + m, i.e. element 15 - m.
    const bool win = unclamped(kt);                       // wave-uniform
    uint2 w4[4];
    if (win) {
      const bf16* run = reinterpret_cast<const bf16*>(
          smem + kBiasOff + (uint32_t)(bs * kPrefillWaves + wave) * kBiasWave + b_read);
#pragma unroll
      for (int k = 0; k < 4; ++k) __builtin_memcpy(&w4[k], run + 4 * k, 8);
    }
    between(pids);
    f32x16 s = f32x16{};
#pragma unroll
    for (int s2 = 0; s2 < 8; ++s2) s = mfma32(kop[s2], qop[s2], s);
    // Element i (S^T row 8 (i / 4) + 4u + i % 4 = key kt + 16u + i) sits at
    // distance D0 - i.
    float bias[16];
    if (win) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        bias[15 - 4 * k] = bf16_lo(w4[k].x);
        bias[14 - 4 * k] = __builtin_bit_cast(float, w4[k].x & 0xffff0000u);
        bias[13 - 4 * k] = bf16_lo(w4[k].y);
        bias[12 - 4 * k] = __builtin_bit_cast(float, w4[k].y & 0xffff0000u);
      }
    } else if (all_clamped(kt)) {
#pragma unroll
      for (int i = 0; i < 16; ++i) bias[i] = bias_cl;
    } else {
      // The tile straddles the clamp: every element's own clamped entry.
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int e = iclamp(D0 - i, 0, R - 1);
        bias[i] = cval ? bf16_lo(bload16(rel_rsrc, row_off + (uint32_t)e * SZ)) : 0.f;
      }
    }
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = fmaf(s[i], P.scale, bias[i]);
    // Mask by select on tiles that cross the window or causal boundary.
    const bool full = (W <= 0 || (wje - 1) - kt < W) && (pbase + wt_lo) - (kt + kN - 1) >= 0;
    if (!full) {                                          // wave-uniform
#pragma unroll
      for (int i = 0; i < 16; ++i) x[i] = (uint32_t)(D0 - i) < wlim ? x[i] : kNegInf;
    }
    float mx = kNegInf;
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, x[i]);
    // A column's first tile with a visible key sets its reference (from
    // -inf: the factor is 0 and the accumulators are still 0); a logit more
    // than kOver above the reference raises it.  A column without a visible
    // key keeps -inf (then P = 0).  Padding columns (no such head or token)
    // never take the branch.
    if (__builtin_amdgcn_ballot_w64(cval && mx > m_ref + kOver)) {   // wave-uniform, rare
      const float mc = fmaxf(mx, xor_lane(mx, 32));
      if (cval && mc > m_ref + kOver) {
        const float alpha = fast_exp2((m_ref - mc) * kLog2e);
#pragma unroll
        for (int dt = 0; dt < kD / 32; ++dt) acc[dt] *= alpha;
        l_run *= alpha;
        m_ref = mc;
      }
    }
    const float mb = m_ref == kNegInf ? 0.f : m_ref * kLog2e;
    // P enters the PV product as two bf16 terms, hi = RNE(P) and lo =
    // RNE(P - hi), whose sum is P to 2^-17 relative; a single bf16 P would
    // move an output by up to 2^-8 of the spread of V.  Exponentials and the
    // hi terms first; the lo terms and the row sum are computed while the
    // hi-term MFMAs run.
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
#pragma unroll
    for (int dt = 0; dt < kD / 32; ++dt)
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
    for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) acc[dt] = mfma32(va[dt][ks], pl[ks], acc[dt]);
  };

  // Append: the tile at kt in stage st straddles the first new token
  // (pbase inside it, so one of its pages was read from the cache).  Each
  // wave replaces its own rows of new keys with the new rows, after its own
  // loads of the tile completed and before the barrier that publishes them.
  auto patch_new = [&](int kt, int st) {
    if (!(kt < pbase && kt + kN > pbase)) return;        // workgroup-uniform
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int key = kt + 16 * i + 4 * wave + (lane >> 4);
      if (key >= pbase && key < je) {
        // Row q0 + key - pbase; k_lane / v_lane hold the slot term of key.
        const int64_t shift = (int64_t)(q0 + kt + 16 * i - pbase) * slot_bytes;
        const uint4 a = *reinterpret_cast<const uint4*>(kn + (uint64_t)((int64_t)k_lane[i] + shift));
        const uint4 c = *reinterpret_cast<const uint4*>(vn + (uint64_t)((int64_t)v_lane + shift));
        const uint32_t blk = (uint32_t)st * kStage + (uint32_t)(2 * wave + i) * 1024u + 16u * (uint32_t)lane;
        *reinterpret_cast<uint4*>(smem + blk + 128u * (uint32_t)wave) = a;
        *reinterpret_cast<uint4*>(smem + blk + kKBytes) = c;
      }
    }
  };

  // ---- software pipeline over key tiles ------------------------------------
  // At the top of each step tile kt sits in K/V stage st and bias stage bs,
  // the next tile's bias is in flight into the stage after; tile kt + N's
  // K/V are issued into the other K/V stage and tile kt + 2N's bias windows
  // into the third bias stage, all while tile kt is computed.  Every wave
  // issues, per step, 4 K/V loads then 3 bias loads, so waiting until at
  // most 3 are in flight completes the next tile's K/V and bias and leaves
  // the one after in flight; one barrier then hands the K/V stage over (each
  // wave's bias region is its own).  Loads past the last tile read nothing,
  // so no load sits under control flow.  Nothing the compiler sees is loaded
  // in the loop outside the rare clamp path, so it adds no waits of its own.
  if constexpr (APPEND) {
    // Store this workgroup's tokens' new K/V rows of head g into the cache
    // (16 chunks of 16 bytes per row and tensor).  Every new key lies below
    // L, so its page is in the sequence's block-table row.
    const int chunks = (tend - t0) * 32;
    for (int c = tid; c < chunks; c += blockDim.x) {
      const int t = t0 + (c >> 5), r = c & 31;
      const bool isv = r >= 16;
      const int key = pbase + t;
      const uint64_t page = (uint32_t)iclamp(
          P.block_table[(int64_t)b * P.max_blocks + imin(key >> 4, last_page)], 0, P.num_blocks - 1);
      const uint64_t dst = page * page_bytes + (uint64_t)(key & 15) * slot_bytes + head_bytes +
                           (uint64_t)(r & 15) * 16u;
      const uint64_t src = (uint64_t)(q0 + t) * slot_bytes + head_bytes + (uint64_t)(r & 15) * 16u;
      const uint4 v = *reinterpret_cast<const uint4*>((isv ? vn : kn) + src);
      *reinterpret_cast<uint4*>(reinterpret_cast<char*>(const_cast<void*>(isv ? P.v : P.k)) + dst) = v;
    }
  }
  int kt = jb & ~15;
  int st = 0, bs = 0;
  issue_kv(kt, 0, page_ids(kt));
  issue_bias(kt, 0);
  issue_bias(kt + kN, 1);
  wait_vmem<3>();
  if constexpr (APPEND) patch_new(kt, 0);
  if (kt < jb) {                                         // workgroup-uniform
    // The first page holds keys before the block's first visible key: their
    // P is 0 for every column, but a non-finite V row would still turn 0 * V
    // into NaN in the PV product, so their V rows are zeroed.  Key k < 16 of
    // the tile sits in LDS row 8 (k >> 2) + (k & 3).
    lds_barrier();
    unsigned char* Vs = smem + kKBytes;
    for (int c = tid; c < (jb - kt) * 16; c += blockDim.x) {
      const int k = c >> 4;
      *reinterpret_cast<uint4*>(Vs + (8 * (k >> 2) + (k & 3)) * 256 + (c & 15) * 16) =
          make_uint4(0u, 0u, 0u, 0u);
    }
  }
  // Page ids are loaded a step ahead and completed before the step's
  // barrier (the empty asm reads them there), so that no wait for them
  // falls between a tile's LDS reads and their use.
  int2 pids_next = page_ids(kt + kN);
  asm volatile("" ::"s"(pids_next.x), "s"(pids_next.y));
  lds_barrier();
  while (true) {
    const int2 pids = pids_next;
    pids_next = page_ids(kt + 2 * kN);
    compute(kt, st, bs, pids, [&](int2 p) {
      issue_kv(kt + kN, st ^ 1, p);
      issue_bias(kt + 2 * kN, bs == 0 ? 2 : bs - 1);
    });
    if (kt + kN >= je) break;                            // workgroup-uniform
    wait_vmem<3>();
    if constexpr (APPEND) patch_new(kt + kN, st ^ 1);
    asm volatile("" ::"s"(pids_next.x), "s"(pids_next.y));
    lds_barrier();
    kt += kN;
    st ^= 1;
    bs = bs == 2 ? 0 : bs + 1;
  }
  // Prefetches past the last tile may be outstanding: drain them before the
  // wave ends.
  __builtin_amdgcn_s_waitcnt(0);

  if (ksplit) {
    // Waves 1..3 hand their accumulators, row sums and references to wave 0
    // through LDS (every wave's loads have landed and its reads are done),
    // which merges them by log-sum-exp weights.
    lds_barrier();
    float* xs = reinterpret_cast<float*>(smem);
    constexpr int kXs = 66 * 64;                          // floats per wave
    if (wave > 0) {
      float* d = xs + (wave - 1) * kXs + lane;
#pragma unroll
      for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) d[(16 * dt + i) * 64] = acc[dt][i];
      d[64 * 64] = m_ref;
      d[65 * 64] = l_run;
    }
    lds_barrier();
    if (wave > 0) return;
    float mw[kPrefillWaves - 1];
    float M = m_ref;
#pragma unroll
    for (int w = 0; w < kPrefillWaves - 1; ++w) {
      mw[w] = xs[w * kXs + 64 * 64 + lane];
      M = fmaxf(M, mw[w]);
    }
    const float e0 = m_ref == kNegInf ? 0.f : fast_exp2((m_ref - M) * kLog2e);
#pragma unroll
    for (int dt = 0; dt < kD / 32; ++dt) acc[dt] *= e0;
    l_run *= e0;
#pragma unroll
    for (int w = 0; w < kPrefillWaves - 1; ++w) {
      const float e = mw[w] == kNegInf ? 0.f : fast_exp2((mw[w] - M) * kLog2e);
      const float* src = xs + w * kXs + lane;
#pragma unroll
      for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[dt][i] += e * src[(16 * dt + i) * 64];
      l_run += e * src[65 * 64];
    }
  }

  if (!wact) return;
  const float lt = l_run + xor_lane(l_run, 32);
  if (!cval) return;
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  bf16* dst = static_cast<bf16*>(P.out) + ((int64_t)(q0 + tc) * hq + h) * kD;
#pragma unroll
  for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const bf16x4 v = {from_f32<bf16>(acc[dt][4 * q4] * inv), from_f32<bf16>(acc[dt][4 * q4 + 1] * inv),
                        from_f32<bf16>(acc[dt][4 * q4 + 2] * inv),
                        from_f32<bf16>(acc[dt][4 * q4 + 3] * inv)};
      *reinterpret_cast<bf16x4*>(dst + 32 * dt + 8 * q4 + 4 * u) = v;
    }
}

}  // namespace

size_t prefill_bf16_lds_bytes() { return (size_t)kLdsBytes; }

hipError_t launch_prefill_bf16(const PrefillParams& p, hipStream_t stream) {
  // Raise the kernel's dynamic LDS limit once per process (thread-safe).
  static std::once_flag once;
  static hipError_t attr = hipSuccess;
  std::call_once(once, [] {
    attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&prefill_bf16_kernel<false>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (attr == hipSuccess)
      attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&prefill_bf16_kernel<true>),
                                 hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  });
  if (attr != hipSuccess) return attr;
  const int64_t total = (int64_t)(p.total_q / p.bq + p.num_seqs) * p.hkv;
  const int64_t grid = ((total + 7) / 8) * 8;
  if (p.k_new != nullptr)
    prefill_bf16_kernel<true><<<dim3((unsigned)grid), dim3(kPrefillWaves * 64),
                                prefill_bf16_lds_bytes(), stream>>>(p);
  else
    prefill_bf16_kernel<false><<<dim3((unsigned)grid), dim3(kPrefillWaves * 64),
                                 prefill_bf16_lds_bytes(), stream>>>(p);
  return hipGetLastError();
}

}  // namespace ira
