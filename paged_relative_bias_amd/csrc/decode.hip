// Single-token decode with split-KV and a log-sum-exp merge, on gfx950.
//
// Operation: the relative-bias attention of the TensorRT-LLM Inkling page
// (section "Architecture") for one new token per sequence at position
// L_b - 1.  The split of each sequence's keys into parts, each producing a
// normalised partial output plus its log-sum-exp, followed by a merge, is
// the split-KV decode the vLLM page describes (section "Changes": up to 128
// splits, with a helper that picks the count).
//
// Work decomposition.  One workgroup per (group of NH adjacent KV heads,
// split, sequence b) with one wave per KV head g (NH = 2 when Hkv is even
// and the dtype is bf16, else 1).  Two-wave workgroups of ~79 KB of LDS put
// two workgroups on a compute unit, each with its own barriers; this
// measured faster than one four-wave workgroup per compute unit (which
// shares one barrier among the four waves) and than single-wave ones.  The G query heads
// of a KV head are its wave's MFMA columns (G <= 16).  A split is a run of
// at most `chunk_tiles` 32-key tiles of the sequence's visible keys, so
// every workgroup of a launch streams about the same number of bytes
// whatever the sequence lengths; sequence b uses ceil(tiles_b /
// chunk_tiles) splits and the workgroups beyond that only mark their
// partials empty.
//
// The kernel is bound by HBM bandwidth; the loop keeps DEPTH tiles of K, V
// and bias loads in flight in a ring of register buffers, all of them
// non-temporal (every byte is read once; measured 3-6% faster than the
// default cache policy):
//   * the page ids of the split are copied once into LDS; a tile's two page
//     ids are one broadcast LDS read, taken to SGPRs;
//   * the NH heads of a workgroup are adjacent in every cache slot, so one
//     wave load covers NH * D contiguous elements of one or more slots;
//     each wave loads 32 / NH slots of the tile for all NH heads;
//   * every K/V load goes through a per-page buffer descriptor whose size
//     stops at the split's last key, so keys past the end (and whole tiles
//     past the last one) read zero without any per-lane test or traffic,
//     and each lane's offset inside a page is a loop constant;
//   * the bias of the tile is, per query head, an aligned run of 40
//     entries of the distance axis loaded as 16-byte chunks (chunks left of
//     the row start read zero through the descriptor bound);
//   * the loads are written to an LDS stage (two stages, alternating by
//     tile, when several waves share it; one barrier per tile), each wave
//     reads its head's K rows as MFMA A operands and its V rows transposed
//     with ds_read_tr16_b64.
// Per tile: S^T[key][head] = K . Q^T (16x16x32 bf16 MFMA); x = scale * S +
// bias; masking by select only on the first and last tile of the split;
// softmax against a per-column reference (the column max of the split's
// first tile, raised, with the wave's accumulators rescaled in registers,
// only on a tile where a logit exceeds it by more than kOver); P as the
// sum of two bf16 terms (hi + lo) with an fp32 row sum; O^T[d][head] +=
// V^T . P^T.  One split writes the output; otherwise each wave writes its
// normalised partial and log-sum-exp, and combine_kernel merges them in
// split order (no atomics).
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

template <typename T, int D, int NH>
struct Decode {
  static constexpr bool kBF16 = sizeof(T) == 2;
  static constexpr int NK = kDecodeKeys;                 // keys per tile
  static constexpr int SZ = (int)sizeof(T);
  static constexpr int VEC = 16 / SZ;                    // elements per 16 B
  static constexpr int CPR = D / VEC;                    // 16-byte chunks per head row
  static constexpr int LPS = NH * CPR;                   // lanes per slot (NH head rows)
  static constexpr int SPI = 64 / LPS;                   // slots per wave load
  static constexpr int SPW = NK / NH;                    // slots each wave loads per tile
  static constexpr int VLD = SPW / SPI;                  // K (and V) loads per wave and tile
  static_assert(LPS <= 64 && SPW % SPI == 0 && 16 % SPI == 0, "load layout");
  static_assert(2 * CPR <= 64, "one K and one V row per wave load");
  static constexpr int KP = D + VEC;                     // K row pitch (elements)
  static constexpr int VSP = kBF16 ? D + 16 : D + 4;     // V row pitch (elements)
  static constexpr int KSTEPS = kBF16 ? D / 32 : D / 4;  // MFMA k-steps per 16 keys
  static constexpr int BW = 40;                          // bias entries staged per head
  static constexpr int BCH = BW / VEC;                   // their 16-byte chunks
  static constexpr int BLD = (kMaxGroup * BCH + 63) / 64;  // bias loads per tile
  static constexpr int DEPTH = kBF16 ? 2 : 1;            // tiles in flight
  static constexpr int NBUF = DEPTH + 1;
  // One wave alone orders its own LDS accesses; several share a tile
  // through two LDS stages and one barrier per tile.
  static constexpr int STAGES = NH > 1 ? 2 : 1;
  using KOp = typename std::conditional<kBF16, bf16x8, float>::type;
  static constexpr size_t k_bytes() { return (size_t)NK * KP * SZ; }
  static constexpr size_t v_bytes() { return (size_t)NK * VSP * SZ; }
  // Rows for every chunk a bias load writes (lanes past the G heads write
  // their zeros to rows nobody reads, so the store needs no condition).
  static constexpr int BROWS = (BLD * 64 + BCH - 1) / BCH;
  static constexpr size_t b_bytes() { return (size_t)BROWS * BW * SZ; }
  // Stage: K of the NH heads, V of the NH heads, then each wave's bias runs.
  static constexpr size_t stage_bytes() { return NH * (k_bytes() + v_bytes() + b_bytes()); }
  static constexpr size_t fixed_lds() { return STAGES * stage_bytes(); }
};

// One wave's loads of a tile: its K and V slots (for all NH heads) and its
// heads' bias runs, all as 16-byte chunks.
template <typename T, int D, int NH>
struct Tile {
  using C = Decode<T, D, NH>;
  uint4 k[C::VLD];
  uint4 v[C::VLD];
  uint4 b[C::BLD];
};

// Orders this wave's LDS accesses for the compiler (the hardware keeps one
// wave's LDS operations in order).
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Workgroup barrier that orders LDS only: in-flight global loads of the
// waves are not waited for.
__device__ __forceinline__ void wg_lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// CLAMP: some visible distance may exceed R - 1 (window or context longer
// than the bias), so bias offsets are clamped per element.
template <typename T, int D, bool CLAMP, int NH>
__global__ void __launch_bounds__(64 * NH) __attribute__((amdgpu_waves_per_eu(1, 1)))
decode_kernel(const DecodeParams P) {
  using C = Decode<T, D, NH>;
  constexpr int NK = C::NK, VSP = C::VSP, CPR = C::CPR, VEC = C::VEC;
  constexpr int LPS = C::LPS, SPI = C::SPI, SPW = C::SPW;
  constexpr int DEPTH = C::DEPTH, NBUF = C::NBUF;
  constexpr uint32_t SZ = sizeof(T);
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  // LDS: STAGES x {K tiles [NH][NK][KP], V tiles [NH][NK][VSP], bias runs
  // [NH][BROWS][BW]}, then the split's page-id table.
  int* pid_lds = reinterpret_cast<int*>(smem + C::fixed_lds());

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = NH > 1 ? __builtin_amdgcn_readfirstlane(tid >> 6) : 0;
  // Workgroup (x, y, z) runs on XCD (x + gridDim.x (y + gridDim.y z)) mod 8.
  // With y the split itself, an XCD would get one parity of split index for
  // every sequence, and the first splits are the ones that are always full;
  // rotating the split by the sequence spreads full and partial splits over
  // the XCDs.
  const int g0 = blockIdx.x * NH, g = g0 + wave;
  const int b = blockIdx.z;
  const int split = (int)((blockIdx.y + blockIdx.z) % gridDim.y);
  const int col = lane & 15, u4 = lane >> 4;
  const int G = P.group, R = P.rel_len, W = P.window;
  const bool cval = col < G;
  const int h = g * G + (cval ? col : 0);
  const int64_t row = (int64_t)b * P.hq + h;
  const bool multi = P.num_splits > 1;

  // Keys of this split: tiles [split * CT, split * CT + ntiles) of the
  // sequence's tiles, which start at the first visible key rounded down to
  // a page boundary.  All of it is uniform over the workgroup.
  const int L = iclamp(P.seq_lens[b], 0, P.max_blocks * 16);
  const int pq = L - 1;                                  // query position
  const int k_lo = W > 0 ? imax(0, L - W) : 0;           // first visible key
  const int kb0 = k_lo & ~15;
  const int seq_tiles = L > kb0 ? (L - kb0 + NK - 1) / NK : 0;
  const int CT = P.chunk_tiles;
  const int ntiles = imin(seq_tiles - split * CT, CT);
  if (ntiles <= 0) {
    // Empty split: an empty partial (lse = -inf), or a zero output row when
    // the sequence has no key at all and there is no merge.
    if (cval) {
      if (multi) {
        if (u4 == 0) P.part_lse[(int64_t)split * P.num_seqs * P.hq + row] = kNegInf;
      } else {
        T* dst = static_cast<T*>(P.out) + row * D;
        for (int d = u4; d < D; d += 4) dst[d] = from_f32<T>(0.f);
      }
    }
    return;
  }
  const int s_lo = kb0 + split * CT * NK;
  const int s_hi = imin(L, s_lo + CT * NK);
  const int v_lo = imax(s_lo, k_lo);                     // visible keys [v_lo, s_hi)

  // Append: the workgroup whose split ends at key L - 1 stores this step's
  // K/V rows of its heads into that key's cache slot, and uses them for the
  // key (its own loads of the slot may see the old contents).  Lanes
  // [0, CPR) hold the K row's 16-byte chunks, lanes [CPR, 2 CPR) the V row's.
  // The rows are loaded here and stored once the page ids are in LDS.
  const bool app = P.k_new != nullptr && s_hi == L;      // uniform
  uint4 new_chunk = make_uint4(0u, 0u, 0u, 0u);
  if (app && lane < 2 * CPR) {
    const bool isv = lane >= CPR;
    const int64_t row = (int64_t)b * P.hkv + g;
    new_chunk = *reinterpret_cast<const uint4*>(static_cast<const char*>(isv ? P.v_new : P.k_new) +
                                                row * D * SZ + (isv ? lane - CPR : lane) * 16);
  }

  // Page ids of the split (and zeros past its end, read by the prefetches
  // beyond the last tile) into LDS.
  const int pg_base = s_lo >> 4;
  const int npg = ((s_hi - 1) >> 4) - pg_base + 1;
  {
    const int seq_pages = (L + 15) >> 4;
    const __amdgpu_buffer_rsrc_t bt_rsrc =
        make_rsrc(P.block_table + (int64_t)b * P.max_blocks, (uint32_t)seq_pages * 4u);
    for (int i = tid; i < P.pid_cap; i += 64 * NH) {
      const uint32_t off = i < npg ? (uint32_t)(pg_base + i) * 4u : kOOB;
      pid_lds[i] = iclamp((int)bload32(bt_rsrc, off), 0, P.num_blocks - 1);
    }
  }

  // Q^T operand (B of the QK MFMA): lane holds head col, d = 32 st + 8 u4 ..
  typename C::KOp qop[C::KSTEPS];
  {
    const T* src = static_cast<const T*>(P.q) + row * D;
    if constexpr (C::kBF16) {
#pragma unroll
      for (int s = 0; s < C::KSTEPS; ++s)
        qop[s] = cval ? *reinterpret_cast<const bf16x8*>(src + 32 * s + 8 * u4) : bf16x8{};
    } else {
#pragma unroll
      for (int s = 0; s < C::KSTEPS; ++s) qop[s] = cval ? src[4 * s + u4] : 0.f;
    }
  }

  // Loop-constant lane offsets.  A page holds 16 slots x Hkv heads x D; the
  // NH heads of the workgroup are adjacent, so one slot of them is NH * D
  // contiguous elements.  Wave load i covers slots wave * SPW + i * SPI +
  // lane / LPS of the tile, head g0 + (lane % LPS) / CPR, 16-byte chunk
  // lane % CPR.
  const uint32_t slot_bytes = (uint32_t)P.hkv * D * SZ;
  const uint32_t page_bytes = 16u * slot_bytes;
  const char* kg = static_cast<const char*>(P.k);
  const char* vg = static_cast<const char*>(P.v);
  uint32_t kv_off[C::VLD];
#pragma unroll
  for (int i = 0; i < C::VLD; ++i)
    kv_off[i] = (uint32_t)((wave * SPW + i * SPI + lane / LPS) & 15) * slot_bytes +
                (uint32_t)g0 * D * SZ + (uint32_t)(lane % LPS) * 16u;
  // Bias: for a tile at kt the keys' distances pq - kt - 31 .. pq - kt lie
  // in an aligned window [w0, w0 + BW) of each head's row; bias load m
  // brings chunk (m * 64 + lane) % BCH of head (m * 64 + lane) / BCH.
  const T* rel_g = static_cast<const T*>(P.rel) + ((int64_t)b * P.hq + (int64_t)g * G) * R;
  const uint32_t rel_bytes = (uint32_t)(G * R) * SZ;
  uint32_t b_off[C::BLD];
#pragma unroll
  for (int m = 0; m < C::BLD; ++m) {
    const int idx = m * 64 + lane, hc = idx / C::BCH, ch = idx % C::BCH;
    b_off[m] = hc < G ? (uint32_t)(hc * R + ch * VEC) * SZ : kOOB;
  }

  // First entry of the bias window of the tile at kt: the smallest
  // distance rounded down to a chunk, or (CLAMP) low enough to reach R - 1.
  auto bias_w0 = [&](int kt) {
    const int w = floor_to(pq - kt - (NK - 1), VEC);
    return CLAMP ? imin(w, floor_to(R - NK, VEC)) : w;
  };

  // Loads of tile t: K rows and bias runs (kb), V rows (vv).  Both flags
  // are constants at every call.
  auto issue = [&](Tile<T, D, NH>& tb, int t, bool kb, bool vv) {
    const int kt = s_lo + t * NK;
    const int2 pp = *reinterpret_cast<const int2*>(pid_lds + 2 * t);
    // Descriptor fields must be scalar: readfirstlane keeps every value
    // below in SGPRs (a VGPR descriptor would need a waterfall loop).
    const uint64_t p0 = (uint32_t)__builtin_amdgcn_readfirstlane(pp.x);
    const uint64_t p1 = (uint32_t)__builtin_amdgcn_readfirstlane(pp.y);
    const uint32_t n0 = sgpr_u32((uint32_t)iclamp(s_hi - kt, 0, 16) * slot_bytes);
    const uint32_t n1 = sgpr_u32((uint32_t)iclamp(s_hi - kt - 16, 0, 16) * slot_bytes);
    const __amdgpu_buffer_rsrc_t k0 = make_rsrc(kg + p0 * page_bytes, n0);
    const __amdgpu_buffer_rsrc_t k1 = make_rsrc(kg + p1 * page_bytes, n1);
    const __amdgpu_buffer_rsrc_t v0 = make_rsrc(vg + p0 * page_bytes, n0);
    const __amdgpu_buffer_rsrc_t v1 = make_rsrc(vg + p1 * page_bytes, n1);
    // Load i reads page (wave * SPW + i * SPI) / 16 of the tile (uniform).
    if (kb) {
#pragma unroll
      for (int i = 0; i < C::VLD; ++i)
        tb.k[i] = bload128_nt(((wave * SPW + i * SPI) >> 4) ? k1 : k0, kv_off[i]);
    }
    if (vv) {
#pragma unroll
      for (int i = 0; i < C::VLD; ++i)
        tb.v[i] = bload128_nt(((wave * SPW + i * SPI) >> 4) ? v1 : v0, kv_off[i]);
    }
    if (!kb) return;
    // Chunks left of a row start (window of the last tile) get a negative
    // offset, out of range as an unsigned value: they read 0.  The offset is
    // kept a full register value so no part of it is folded into the
    // instruction's unsigned offset field.
    const __amdgpu_buffer_rsrc_t rr = make_rsrc(rel_g, sgpr_u32(t < ntiles ? rel_bytes : 0u));
    const uint32_t wsh = (uint32_t)bias_w0(kt) * SZ;
#pragma unroll
    for (int m = 0; m < C::BLD; ++m) {
      uint32_t off = b_off[m] + wsh;
      asm volatile("" : "+v"(off));
      tb.b[m] = bload128_nt(rr, off);
    }
  };

  // The wave's loads of a tile into LDS stage st: its K and V slots of all
  // NH heads, and its own bias runs.
  auto stage_tile = [&](const Tile<T, D, NH>& tb, int st) {
    unsigned char* base = smem + (size_t)st * C::stage_bytes();
    T* Ks = reinterpret_cast<T*>(base);
    T* Vs = reinterpret_cast<T*>(base + NH * C::k_bytes());
    T* Bs = reinterpret_cast<T*>(base + NH * (C::k_bytes() + C::v_bytes()) + wave * C::b_bytes());
    const int hh = (lane % LPS) / CPR, chunk = (lane % CPR) * VEC;
#pragma unroll
    for (int i = 0; i < C::VLD; ++i) {
      const int key = wave * SPW + i * SPI + lane / LPS;
      *reinterpret_cast<uint4*>(Ks + (hh * NK + key) * C::KP + chunk) = tb.k[i];
      *reinterpret_cast<uint4*>(Vs + (hh * NK + key) * VSP + chunk) = tb.v[i];
    }
#pragma unroll
    for (int m = 0; m < C::BLD; ++m) {
      const int idx = m * 64 + lane;
      *reinterpret_cast<uint4*>(Bs + (idx / C::BCH) * C::BW + (idx % C::BCH) * VEC) = tb.b[m];
    }
  };

  f32x4 acc[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) acc[dt] = f32x4{};
  // Softmax reference (the four lanes of a column agree on it): the column
  // max of the split's first tile, which always holds a visible key.  Later
  // logits may exceed it; P = exp(x - m_ref) stays far from overflow while
  // they exceed it by at most kOver.  On a tile where a logit exceeds it by
  // more, the column's reference becomes that tile's column max and its
  // accumulators and row sum are multiplied by exp(old - new), in registers
  // and only on that tile.
  float m_ref = kNegInf, l_run = 0.f;

  // Tile t of this wave's head from LDS stage st.
  auto compute = [&](int t, int st) {
    const int kt = s_lo + t * NK;
    const unsigned char* base = smem + (size_t)st * C::stage_bytes();
    const T* Ks = reinterpret_cast<const T*>(base) + wave * NK * C::KP;
    const T* Vs = reinterpret_cast<const T*>(base + NH * C::k_bytes()) + wave * NK * VSP;
    const T* Bs = reinterpret_cast<const T*>(base + NH * (C::k_bytes() + C::v_bytes()) +
                                             wave * C::b_bytes());
    // S^T blocks: lane holds head col, keys kt + 16 blk + 4 u4 + i.  A
    // operand: key 16 blk + col, d = 32 st + 8 u4 .. (bf16) or 4 st + u4.
    f32x4 s[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      s[blk] = f32x4{};
      const T* kr = Ks + (16 * blk + col) * C::KP;
#pragma unroll
      for (int k = 0; k < C::KSTEPS; ++k) {
        if constexpr (C::kBF16)
          s[blk] = mfma16(*reinterpret_cast<const bf16x8*>(kr + 32 * k + 8 * u4), qop[k], s[blk]);
        else
          s[blk] = mfma16(kr[4 * k + u4], qop[k], s[blk]);
      }
    }
    // Bias of key c = 16 blk + i (i < 4) of the lane: distance pq - kt -
    // 4 u4 - c, entry (distance - w0) of the head's staged run.
    float bias[8];
    {
      const T* br = Bs + col * C::BW;
      const int e3 = pq - kt - 4 * u4 - 3 - bias_w0(kt);   // entry of c = 3
      if constexpr (CLAMP) {
        const int w0 = bias_w0(kt);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int d = pq - kt - 4 * u4 - (16 * (i >> 2) + (i & 3));
          bias[i] = to_f32(br[iclamp(imin(d, R - 1) - w0, 0, C::BW - 1)]);
        }
      } else if constexpr (C::kBF16) {
        // Four consecutive entries per block: c = 3, 2, 1, 0 upwards.
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
          const int e = iclamp(e3 - 16 * blk, 0, C::BW - 4);
          uint2 r;
          __builtin_memcpy(&r, br + e, 8);
          bias[4 * blk + 3] = __builtin_bit_cast(float, r.x << 16);
          bias[4 * blk + 2] = __builtin_bit_cast(float, r.x & 0xffff0000u);
          bias[4 * blk + 1] = __builtin_bit_cast(float, r.y << 16);
          bias[4 * blk + 0] = __builtin_bit_cast(float, r.y & 0xffff0000u);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i)
          bias[i] = to_f32(br[iclamp(e3 + 3 - (16 * (i >> 2) + (i & 3)), 0, C::BW - 1)]);
      }
    }
    float x[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = fmaf(s[i >> 2][i & 3], P.scale, bias[i]);
    if (kt < v_lo || kt + NK > s_hi) {                   // uniform: edge tile
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int j = kt + 16 * (i >> 2) + 4 * u4 + (i & 3);
        x[i] = (uint32_t)(j - v_lo) < (uint32_t)(s_hi - v_lo) ? x[i] : kNegInf;
      }
    }
    const float mx = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                           fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
    // The first tile sets the reference (from -inf: the factor is 0 and the
    // accumulators are still 0); a logit more than kOver above it raises it.
    // Padding columns (no such head) never take the branch.
    if (__builtin_amdgcn_ballot_w64(cval && mx > m_ref + kOver)) {   // wave-uniform, rare
      const float m4 = fmaxf(mx, xor_lane(mx, 16));
      const float mc = fmaxf(m4, xor_lane(m4, 32));
      if (cval && mc > m_ref + kOver) {
        const float alpha = fast_exp2((m_ref - mc) * kLog2e);
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) acc[dt] *= alpha;
        l_run *= alpha;
        m_ref = mc;
      }
    }
    // P = exp(x - m_ref), and O^T += V^T . P^T.
    const float mb = m_ref == kNegInf ? 0.f : m_ref * kLog2e;
    if constexpr (C::kBF16) {
      // P enters the PV product as two bf16 terms, hi = RNE(P) and lo =
      // RNE(P - hi), whose sum is P to 2^-17 relative; a single bf16 P would
      // move an output by up to 2^-9 of the spread of V.
      bf16x8 ph, pl;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float pf = fast_exp2(fmaf(x[i], kLog2e, -mb));
        const bf16 h = from_f32<bf16>(pf);
        ph[i] = h;
        pl[i] = from_f32<bf16>(pf - (float)h);
        l_run += pf;
      }
      // V^T operand: contraction slots (u4, e) hold keys 4 u4 + e (e < 4)
      // and 16 + 4 u4 + e - 4 (e >= 4), the keys of ph's and pl's slots.  A
      // transposed read: lane jj of a 16-lane group points at key
      // 4 u4 + jj / 4, columns 4 (jj % 4) .. +3; lane i receives column i
      // of those four keys.
      const int jj = lane & 15;
      const T* r0 = Vs + (4 * u4 + (jj >> 2)) * VSP + 4 * (jj & 3);
      const T* r1 = r0 + 16 * VSP;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) {
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(r0 + 16 * dt));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(r1 + 16 * dt));
        const i16x8 a16 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        acc[dt] = mfma16(__builtin_bit_cast(bf16x8, a16), ph, acc[dt]);
        acc[dt] = mfma16(__builtin_bit_cast(bf16x8, a16), pl, acc[dt]);
      }
    } else {
      float pf[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        pf[i] = fast_exp2(fmaf(x[i], kLog2e, -mb));
        l_run += pf[i];
      }
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) {
        const T* vc = Vs + 16 * dt + col;
#pragma unroll
        for (int i = 0; i < 8; ++i)
          acc[dt] = mfma16(vc[(16 * (i >> 2) + 4 * u4 + (i & 3)) * VSP], pf[i], acc[dt]);
      }
    }
  };

  // Page ids visible to every wave.
  if constexpr (NH > 1) wg_lds_barrier(); else wave_lds_fence();
  if (app && lane < 2 * CPR) {
    const bool isv = lane >= CPR;
    const int64_t slot = (int64_t)pid_lds[((L - 1) >> 4) - pg_base] * 16 + ((L - 1) & 15);
    char* dst = static_cast<char*>(const_cast<void*>(isv ? P.v : P.k)) +
                (slot * P.hkv + g) * D * SZ + (isv ? lane - CPR : lane) * 16;
    *reinterpret_cast<uint4*>(dst) = new_chunk;
  }
  // Ring of NBUF tile buffers: tile t is staged from buffer t % NBUF while
  // tiles t+1 .. t+DEPTH are in flight.  The K rows and bias runs of tile
  // t+DEPTH are issued before tile t is staged, its V rows after tile t is
  // computed, so that a wave's K and V requests for the same slots do not
  // reach memory together.  Loads past the last tile read nothing
  // (zero-size descriptors), so no load sits under control flow.
  // With several waves, tile t goes to LDS stage t % 2: the barrier after
  // staging it also tells every wave that all have finished computing tile
  // t - 1, whose stage the next tile reuses.
  Tile<T, D, NH> tb[NBUF];
  {
#pragma unroll
    for (int i = 0; i < DEPTH; ++i) issue(tb[i], i, true, true);
    for (int t0 = 0;; t0 += NBUF) {
#pragma unroll
      for (int r = 0; r < NBUF; ++r) {
        const int t = t0 + r;
        issue(tb[(r + DEPTH) % NBUF], t + DEPTH, true, false);
        const int st = C::STAGES > 1 ? (t & 1) : 0;
        if constexpr (NH == 1) wave_lds_fence();
        if (t == 0 && s_lo < k_lo) {                     // uniform: split 0 only
          // Keys of the first page before the first visible key: their P is
          // 0, but a non-finite V row would still turn 0 * V into NaN in
          // the PV product, so their V rows are staged as zeros.
#pragma unroll
          for (int i = 0; i < C::VLD; ++i)
            if (s_lo + wave * SPW + i * SPI + lane / LPS < k_lo) tb[r].v[i] = make_uint4(0u, 0u, 0u, 0u);
        }
        stage_tile(tb[r], st);
        if constexpr (NH > 1) wg_lds_barrier(); else wave_lds_fence();
        if (app && t == ntiles - 1) {                    // uniform: holds key L - 1
          // Only this wave reads its head's rows, so no barrier is needed.
          const int key = L - 1 - (s_lo + t * NK);
          unsigned char* base = smem + (size_t)st * C::stage_bytes();
          if (lane < CPR) {
            T* Ks = reinterpret_cast<T*>(base) + (wave * NK + key) * C::KP + lane * VEC;
            *reinterpret_cast<uint4*>(Ks) = new_chunk;
          } else if (lane < 2 * CPR) {
            T* Vs = reinterpret_cast<T*>(base + NH * C::k_bytes()) + (wave * NK + key) * VSP +
                    (lane - CPR) * VEC;
            *reinterpret_cast<uint4*>(Vs) = new_chunk;
          }
          wave_lds_fence();
        }
        compute(t, st);
        issue(tb[(r + DEPTH) % NBUF], t + DEPTH, false, true);
        if (t + 1 >= ntiles) goto done;
      }
    }
  done:
    // Loads past the last tile may still be outstanding: drain them before
    // the wave ends.
    __builtin_amdgcn_s_waitcnt(0);
  }
  l_run += xor_lane(l_run, 16);
  l_run += xor_lane(l_run, 32);
  if (!cval) return;
  // acc[dt][i] = O[head col][d = 16 dt + 4 u4 + i] (unnormalised).
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  if (!multi) {
    T* dst = static_cast<T*>(P.out) + row * D + 4 * u4;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      if constexpr (C::kBF16) {
        const bf16x4 v = {from_f32<bf16>(acc[dt][0] * inv), from_f32<bf16>(acc[dt][1] * inv),
                          from_f32<bf16>(acc[dt][2] * inv), from_f32<bf16>(acc[dt][3] * inv)};
        *reinterpret_cast<bf16x4*>(dst + 16 * dt) = v;
      } else {
        *reinterpret_cast<f32x4*>(dst + 16 * dt) = acc[dt] * inv;
      }
    }
  } else {
    const int64_t prow = (int64_t)split * P.num_seqs * P.hq + row;
    float* po = P.part_o + prow * D + 4 * u4;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) *reinterpret_cast<f32x4*>(po + 16 * dt) = acc[dt] * inv;
    if (u4 == 0)
      P.part_lse[prow] = l_run > 0.f ? m_ref + __logf(l_run) : kNegInf;
  }
}

// One wave per (sequence, head) row.  The split log-sum-exps are read one
// per lane (two for more than 64 splits), their max and the weight sum are
// wave reductions, and each split's weight reaches the whole wave as a
// scalar, so that empty splits (lse = -inf) skip their row with a uniform
// branch.  Lane l accumulates d = l + 64 k; the partial rows of up to 8
// splits are in flight at once.  The order of the sum is fixed (split
// order), with no atomics.
template <typename T, int D>
__global__ void __launch_bounds__(256)
combine_kernel(const CombineParams P) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= P.rows) return;
  const int lane = threadIdx.x & 63;
  constexpr int PER = D / 64;
  const int S = P.num_splits;
  const float l0 = lane < S ? P.part_lse[(int64_t)lane * P.rows + row] : kNegInf;
  const float l1 = lane + 64 < S ? P.part_lse[(int64_t)(lane + 64) * P.rows + row] : kNegInf;
  float M = fmaxf(l0, l1);
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) M = fmaxf(M, xor_lane(M, m));
  const float w0 = M == kNegInf || l0 == kNegInf ? 0.f : expf(l0 - M);
  const float w1 = M == kNegInf || l1 == kNegInf ? 0.f : expf(l1 - M);
  float den = w0 + w1;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) den += xor_lane(den, m);
  float num[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) num[k] = 0.f;
  const float* po = P.part_o + (int64_t)row * D + lane;
  const int64_t split_stride = (int64_t)P.rows * D;
  for (int s0 = 0; s0 < S; s0 += 8) {
    float v[8][PER];
    float w[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int s = s0 + j;
      // The split's weight, from lane s % 64 of w0 (s < 64) or w1.
      const float wl = s < 64 ? w0 : w1;
      w[j] = s < S ? __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                                   __builtin_bit_cast(int, wl), s & 63))
                   : 0.f;
#pragma unroll
      for (int k = 0; k < PER; ++k)
        v[j][k] = w[j] != 0.f ? po[s * split_stride + 64 * k] : 0.f;   // uniform branch
    }
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int k = 0; k < PER; ++k) num[k] += w[j] * v[j][k];
  }
  T* dst = static_cast<T*>(P.out) + (int64_t)row * D;
#pragma unroll
  for (int k = 0; k < PER; ++k)
    dst[lane + 64 * k] = from_f32<T>(den > 0.f ? num[k] / den : 0.f);
}

template <typename T, int D>
size_t decode_lds_t(const DecodeParams& p) {
  size_t fixed = Decode<T, D, 1>::fixed_lds();
  if constexpr (sizeof(T) == 2) {
    if (p.heads_per_wg == 2) fixed = Decode<T, D, 2>::fixed_lds();
  }
  return fixed + (size_t)p.pid_cap * 4;
}

template <typename T, int D, bool CLAMP, int NH>
hipError_t launch_decode_c(const DecodeParams& p, hipStream_t stream) {
  // Raise the kernel's dynamic LDS limit once per process (thread-safe).
  static std::once_flag once;
  static hipError_t attr = hipSuccess;
  std::call_once(once, [] {
    attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&decode_kernel<T, D, CLAMP, NH>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  });
  if (attr != hipSuccess) return attr;
  const dim3 grid(p.hkv / NH, p.num_splits, p.num_seqs);
  decode_kernel<T, D, CLAMP, NH><<<grid, dim3(64 * NH), decode_lds_t<T, D>(p), stream>>>(p);
  return hipGetLastError();
}

template <typename T, int D, int NH>
hipError_t launch_decode_h(const DecodeParams& p, hipStream_t stream) {
  return p.clamp ? launch_decode_c<T, D, true, NH>(p, stream)
                 : launch_decode_c<T, D, false, NH>(p, stream);
}

template <typename T, int D>
hipError_t launch_decode_t(const DecodeParams& p, hipStream_t stream) {
  if constexpr (sizeof(T) == 2) {
    if (p.heads_per_wg == 2) return launch_decode_h<T, D, 2>(p, stream);
  }
  if (p.heads_per_wg != 1) return hipErrorInvalidValue;
  return launch_decode_h<T, D, 1>(p, stream);
}

template <typename T, int D>
hipError_t launch_combine_t(const CombineParams& p, hipStream_t stream) {
  const unsigned blocks = (unsigned)((p.rows + 3) / 4);
  combine_kernel<T, D><<<dim3(blocks), dim3(256), 0, stream>>>(p);
  return hipGetLastError();
}

// Device-resident split workspace for callers that cannot allocate
// (inkling_rel_attn_decode_noalloc): partial outputs and log-sum-exps of the
// split-KV decode.  Each GPU the library runs on holds its own copy until
// the process ends; every call on that GPU shares it.
constexpr size_t kScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

}  // namespace

size_t decode_scratch_bytes() { return kScratchBytes; }

hipError_t decode_scratch(int device, void** ptr) {
  *ptr = nullptr;
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  // Once per device, with that device current: the array's address on that
  // device (the name itself is only a host-side stand-in).
  std::call_once(g_scratch_once[device], [device] {
    int prev = -1;
    hipError_t e = hipGetDevice(&prev);
    if (e == hipSuccess && prev != device) e = hipSetDevice(device);
    void* p = nullptr;
    if (e == hipSuccess) e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (prev >= 0 && prev != device) (void)hipSetDevice(prev);
    g_scratch_err[device] = e;
    g_scratch_ptr[device] = e == hipSuccess ? p : nullptr;
  });
  *ptr = g_scratch_ptr[device];
  return g_scratch_err[device];
}

size_t decode_lds_bytes(const DecodeParams& p, int dtype, int head_dim) {
  if (dtype == 0)
    return head_dim == 64 ? decode_lds_t<bf16, 64>(p) : decode_lds_t<bf16, 128>(p);
  return head_dim == 64 ? decode_lds_t<float, 64>(p) : decode_lds_t<float, 128>(p);
}

hipError_t launch_decode(const DecodeParams& p, int dtype, int head_dim, hipStream_t stream) {
  if (dtype == 0)
    return head_dim == 64 ? launch_decode_t<bf16, 64>(p, stream)
                          : launch_decode_t<bf16, 128>(p, stream);
  return head_dim == 64 ? launch_decode_t<float, 64>(p, stream)
                        : launch_decode_t<float, 128>(p, stream);
}

hipError_t launch_combine(const CombineParams& p, int dtype, int head_dim, hipStream_t stream) {
  if (dtype == 0)
    return head_dim == 64 ? launch_combine_t<bf16, 64>(p, stream)
                          : launch_combine_t<bf16, 128>(p, stream);
  return head_dim == 64 ? launch_combine_t<float, 64>(p, stream)
                        : launch_combine_t<float, 128>(p, stream);
}

}  // namespace ira
