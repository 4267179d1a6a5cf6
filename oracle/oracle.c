/*
 * fp64 CPU oracle for paged relative-bias attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the HIP library in paged_relative_bias_amd/.
 *
 * What it computes (TensorRT-LLM Inkling page, section "Architecture"): the
 * model has no rotary embedding; position enters only through a learned
 * bias, one value per (query token, head, relative distance), added to the
 * attention logits before the softmax.  Local layers attend over a sliding
 * window of 512 keys, global layers over the full causal prefix, and the
 * query heads share grouped KV heads.  The same page asks reviewers to check
 * the bias shapes, the sliding-window mask and the handling of cache pages,
 * and the vLLM page (section "Purpose") notes that vLLM's attention for this
 * model reads keys and values from the paged cache in every configuration.
 * The bias is added to the QK^T logit after the scale is applied.
 *
 * Plain definition, evaluated independently for every (query row i, head h):
 *
 *   b     = the sequence owning row i  (cu_q_lens[b] <= i < cu_q_lens[b+1])
 *   n_b   = cu_q_lens[b+1] - cu_q_lens[b]        new tokens of sequence b
 *   L_b   = seq_lens[b]                          keys, including the new ones
 *   p     = L_b - n_b + (i - cu_q_lens[b])       logical position of row i
 *   g     = h / (Hq / Hkv)                       grouped KV head
 *   for every logical key j in [0, L_b):
 *       d = p - j
 *       visible(j) = d >= 0 and (window <= 0 or d < window)
 *       K_j = k_cache[block_table[b][j / bs]][j % bs][g][:]   (V_j likewise)
 *       s_j = scale * <q[i][h], K_j> + rel[i][h][min(d, R - 1)]
 *   M = max over visible s_j,  Z = sum over visible exp(s_j - M)
 *   out[i][h][:] = sum over visible exp(s_j - M) / Z * V_j
 *   lse[i][h]    = M + ln Z
 *
 * Readings where the pages are silent: the window holds W keys including the
 * query itself (d < W);
 * the distance index is clamped to R - 1; query position is bottom-right
 * aligned (p = L_b - n_b + t); query head h uses KV head h / (Hq / Hkv); an
 * empty visible set gives out = 0 and lse = -inf.
 *
 * Inputs are read exactly (bfloat16 widened to float by its definition: the
 * 16 stored bits are the high half of an IEEE binary32) and every operation
 * is done in double with the host libm exp/log and straight summation in key
 * order.  Only visible keys and bias entries are read.  Rows are independent
 * and evaluated in parallel with OpenMP.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_BF16 = 0, OR_FP32 = 1 };

static double rd(const void *base, int dtype, int64_t idx) {
  if (dtype == OR_BF16) {
    uint32_t u = (uint32_t)((const uint16_t *)base)[idx] << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
  }
  return (double)((const float *)base)[idx];
}

/* Sequence owning packed query row i: cu_q_lens is non-decreasing. */
static int owner(const int32_t *cu, int nseq, int64_t i) {
  int lo = 0, hi = nseq - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) / 2;
    if ((int64_t)cu[mid] <= i) lo = mid; else hi = mid - 1;
  }
  return lo; /* the last sequence starting at or before i owns it */
}

typedef struct {
  int32_t num_seqs, num_q_heads, num_kv_heads, head_dim, block_size;
  int32_t max_blocks_per_seq, rel_len, total_q;
} oracle_dims_t;

/*
 * Attention for a list of (row, head) pairs.
 *   rows:   flat indices i * Hq + h to evaluate; NULL means all total_q * Hq.
 *   key_lo, key_hi: optional per-sequence logical key range [lo, hi) that is
 *           intersected with the visible set (NULL = no restriction).  Used to
 *           form the partial results of a split of the key range.
 *   out:    [nrows, head_dim] doubles;  lse: [nrows] doubles (may be NULL).
 * Returns 0, or -1 on an argument the definition cannot evaluate.
 */
int oracle_attention(int dtype, const void *q, const void *k_cache,
                     const void *v_cache, const int32_t *block_table,
                     const int32_t *seq_lens, const int32_t *cu_q_lens,
                     const void *rel_logits, int32_t window, double scale,
                     const oracle_dims_t *dm, const int32_t *key_lo,
                     const int32_t *key_hi, const int64_t *rows, int64_t nrows,
                     double *out, double *lse, int32_t threads) {
  const int B = dm->num_seqs, Hq = dm->num_q_heads, Hkv = dm->num_kv_heads;
  const int D = dm->head_dim, bs = dm->block_size, R = dm->rel_len;
  if (B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || D <= 0 || bs <= 0 || R <= 0)
    return -1;
  const int G = Hq / Hkv;
  if (rows == NULL) nrows = (int64_t)dm->total_q * Hq;
  int maxL = 0;
  for (int b = 0; b < B; ++b) maxL = seq_lens[b] > maxL ? seq_lens[b] : maxL;
#ifdef _OPENMP
  if (threads > 0) omp_set_num_threads(threads);
#else
  (void)threads;
#endif
  int bad = 0;
#pragma omp parallel reduction(| : bad)
  {
    double *s = (double *)malloc(sizeof(double) * (size_t)(maxL > 0 ? maxL : 1));
    unsigned char *vis = (unsigned char *)malloc((size_t)(maxL > 0 ? maxL : 1));
    double *acc = (double *)malloc(sizeof(double) * (size_t)D);
#pragma omp for schedule(dynamic, 16)
    for (int64_t r = 0; r < nrows; ++r) {
      const int64_t flat = rows ? rows[r] : r;
      const int64_t i = flat / Hq;
      const int h = (int)(flat % Hq);
      double *o = out + r * D;
      if (i < 0 || i >= dm->total_q) { bad = 1; continue; }
      const int b = owner(cu_q_lens, B, i);
      const int n_b = cu_q_lens[b + 1] - cu_q_lens[b];
      const int L = seq_lens[b];
      const int p = L - n_b + (int)(i - cu_q_lens[b]);
      const int g = h / G;
      const int lo = key_lo ? key_lo[b] : 0;
      const int hi = key_hi ? key_hi[b] : L;
      const int64_t qoff = (i * Hq + h) * (int64_t)D;
      const int64_t roff = (i * Hq + h) * (int64_t)R;
      double M = -INFINITY;
      int any = 0;
      for (int j = 0; j < L; ++j) {
        const int d = p - j;
        vis[j] = (d >= 0) && (window <= 0 || d < window) && j >= lo && j < hi;
        if (!vis[j]) continue;
        const int32_t blk = block_table[(int64_t)b * dm->max_blocks_per_seq + j / bs];
        const int64_t koff = (((int64_t)blk * bs + j % bs) * Hkv + g) * D;
        double dot = 0.0;
        for (int k = 0; k < D; ++k)
          dot += rd(q, dtype, qoff + k) * rd(k_cache, dtype, koff + k);
        const int di = d < R - 1 ? d : R - 1;
        s[j] = scale * dot + rd(rel_logits, dtype, roff + di);
        if (s[j] > M) M = s[j];
        any = 1;
      }
      for (int k = 0; k < D; ++k) acc[k] = 0.0;
      if (!any) {
        for (int k = 0; k < D; ++k) o[k] = 0.0;
        if (lse) lse[r] = -INFINITY;
        continue;
      }
      double Z = 0.0;
      for (int j = 0; j < L; ++j) {
        if (!vis[j]) continue;
        const double w = exp(s[j] - M);
        Z += w;
        const int32_t blk = block_table[(int64_t)b * dm->max_blocks_per_seq + j / bs];
        const int64_t voff = (((int64_t)blk * bs + j % bs) * Hkv + g) * D;
        for (int k = 0; k < D; ++k) acc[k] += w * rd(v_cache, dtype, voff + k);
      }
      for (int k = 0; k < D; ++k) o[k] = acc[k] / Z;
      if (lse) lse[r] = M + log(Z);
    }
    free(s);
    free(vis);
    free(acc);
  }
  return bad ? -1 : 0;
}

/*
 * Merge of partial results over a partition of the key range (the split-KV
 * decode of the vLLM page, section "Changes": FA4 splits the keys into up to
 * 128 parts).  Each part s carries its normalised output o_s and its
 * log-sum-exp lse_s.  With M = max_s lse_s and w_s = exp(lse_s - M), the
 * whole-range result is sum_s w_s o_s / sum_s w_s and lse = M + ln sum_s w_s.
 * Parts with lse_s = -inf carry no keys and weigh zero.
 *   o_s: [nsplit, nrows, D];  lse_s: [nsplit, nrows];  out: [nrows, D].
 */
void oracle_lse_combine(int32_t nsplit, int64_t nrows, int32_t D,
                        const double *o_s, const double *lse_s, double *out,
                        double *lse) {
  for (int64_t r = 0; r < nrows; ++r) {
    double M = -INFINITY;
    for (int s = 0; s < nsplit; ++s) {
      const double x = lse_s[(int64_t)s * nrows + r];
      if (x > M) M = x;
    }
    double *o = out + r * D;
    for (int k = 0; k < D; ++k) o[k] = 0.0;
    if (M == -INFINITY) {
      if (lse) lse[r] = -INFINITY;
      continue;
    }
    double W = 0.0;
    for (int s = 0; s < nsplit; ++s) {
      const double x = lse_s[(int64_t)s * nrows + r];
      if (x == -INFINITY) continue;
      const double w = exp(x - M);
      W += w;
      const double *os = o_s + ((int64_t)s * nrows + r) * D;
      for (int k = 0; k < D; ++k) o[k] += w * os[k];
    }
    for (int k = 0; k < D; ++k) o[k] /= W;
    if (lse) lse[r] = M + log(W);
  }
}

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
