/*
 * oracle.c -- plain CPU reference of the MoE-layer forward.  See oracle.h.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the tests, the smoke entry point and the
 * benchmark's CPU-baseline leg; never by the HIP library.
 *
 * Readings of the pages adopted here (the pages are silent on these points):
 *  - logits: fp64 accumulation left to right over the hidden index, router bias
 *    added last in fp64, one rounding to fp32;
 *  - ties in any ranking go to the lower expert (or group) index;
 *  - capacity = ceil(cf * N * k / E) (the mean load times the factor), and
 *    slots are admitted in token order (or, on request, first choices of all
 *    tokens before any second choice: the top-2 router of GShard);
 *  - a dropped slot contributes nothing and the remaining weights are not
 *    renormalised; the layer output includes the residual;
 *  - the group score is the maximum biased selection score in the group;
 *  - H, O and y round to the layer dtype (bf16: round-to-nearest-even).
 */
#include "oracle.h"

#include <float.h>
#include <limits.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static int32_t g_threads = 1;

void oracle_set_threads(int32_t n) { g_threads = n < 1 ? 1 : n; }
int32_t oracle_get_threads(void) { return g_threads; }

/* ---------------------------------------------------------------- dtypes -- */

static double bf16_bits_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

static double elem(const void* p, int32_t dtype, size_t i) {
  if (dtype == 0) return (double)((const float*)p)[i];
  return bf16_bits_to_double(((const uint16_t*)p)[i]);
}

/* Round an fp64 value to bf16 with a single round-to-nearest-even step.
 * bf16 carries 8 significant bits and fp32's exponent range; below 2^-126 the
 * spacing stays 2^-133 (subnormals). */
static uint16_t double_to_bf16_bits(double v) {
  if (isnan(v)) return (uint16_t)0x7fc0;
  if (v == 0.0) return signbit(v) ? (uint16_t)0x8000 : (uint16_t)0x0000;
  int ex;
  (void)frexp(fabs(v), &ex);      /* |v| = m * 2^ex with m in [0.5, 1) */
  int q_exp = ex - 8;             /* spacing of 8-bit significands */
  if (q_exp < -133) q_exp = -133;
  double q = rint(ldexp(fabs(v), -q_exp)); /* default rounding: ties to even */
  double r = ldexp(q, q_exp);
  const double bf16_max = ldexp(255.0, 120); /* (2 - 2^-7) * 2^127 */
  float f = r > bf16_max ? INFINITY : (float)r; /* exact: r is a bf16 value */
  if (signbit(v)) f = -f;
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return (uint16_t)(u >> 16);
}

static void store(void* p, int32_t dtype, size_t i, double v) {
  if (dtype == 0)
    ((float*)p)[i] = (float)v;
  else
    ((uint16_t*)p)[i] = double_to_bf16_bits(v);
}

static int dtype_ok(int32_t dtype) { return dtype == 0 || dtype == 1; }

static int desc_ok(const oracle_desc* d) {
  if (!d) return 0;
  if (d->num_tokens < 0 || d->hidden < 1 || d->num_experts < 1) return 0;
  if (d->top_k < 1 || d->top_k > d->num_experts) return 0;
  if (d->num_ranks < 1 || d->num_experts % d->num_ranks != 0) return 0;
  if (d->num_groups < 1 || d->num_experts % d->num_groups != 0) return 0;
  if (d->topk_groups < 1 || d->topk_groups > d->num_groups) return 0;
  if ((int64_t)d->topk_groups * (d->num_experts / d->num_groups) < d->top_k) return 0;
  if (d->score_fn < 0 || d->score_fn > 2) return 0;
  if (!dtype_ok(d->dtype)) return 0;
  return 1;
}

/* ---------------------------------------------------------------- route --- */

/* Router scores: the router is a linear layer over the hidden state
 * ([EP-glossary] "How tokens travel between GPUs", step 1 and the routing
 * snippet, where the router is a Linear(hidden, num_experts)).
 * Fixed summation: acc starts at 0 and adds x[t,i]*w[e,i] for i = 0..d-1 in
 * order, in fp64.  Each product of two fp32 (or bf16) values is exact in fp64,
 * so each step is the same as a fused multiply-add.  The bias is added last,
 * then the sum is rounded once to fp32. */
int oracle_logits(const oracle_desc* desc, const void* x, const void* w,
                  const float* router_bias, float* z) {
  if (!desc_ok(desc) || (desc->num_tokens > 0 && (!x || !w || !z))) return -1;
  const int32_t N = desc->num_tokens, d = desc->hidden, E = desc->num_experts;
  double* wd = (double*)malloc(sizeof(double) * (size_t)E * d);
  if (!wd) return -1;
  for (size_t i = 0; i < (size_t)E * d; ++i) wd[i] = elem(w, desc->dtype, i);

  int failed = 0;
#pragma omp parallel num_threads(g_threads)
  {
    double* xd = (double*)malloc(sizeof(double) * (size_t)d);
    if (!xd) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(static)
    for (int32_t t = 0; t < N; ++t) {
      if (!xd) continue;
      for (int32_t i = 0; i < d; ++i) xd[i] = elem(x, desc->dtype, (size_t)t * d + i);
      for (int32_t e = 0; e < E; ++e) {
        const double* we = wd + (size_t)e * d;
        double acc = 0.0;
        for (int32_t i = 0; i < d; ++i) acc = acc + xd[i] * we[i];
        if (router_bias) acc = acc + (double)router_bias[e];
        z[(size_t)t * E + e] = (float)acc;
      }
    }
    free(xd);
  }
  free(wd);
  return failed ? -1 : 0;
}

/* DeepSeek-V3-style affinity: the logistic function of the logit, evaluated in
 * fp64 and rounded once to fp32. */
static float sigmoid_affinity(float z) { return (float)(1.0 / (1.0 + exp(-(double)z))); }

/* Is (sa, a) ranked before (sb, b)?  Higher score first, lower index on ties. */
static int ranks_before(float sa, int32_t a, float sb, int32_t b) {
  return sa > sb || (sa == sb && a < b);
}

/* Selection and weights for one token.
 *  - selection score: the router score plus the per-expert selection bias,
 *    which only affects which experts are chosen ([EP-glossary] "Load
 *    balancing and capacity", bias-based balancing bullet);
 *  - score function: softmax over the selected logits (top-2 GShard / Mixtral
 *    style), softmax over all experts (top-1 Switch, [MLSys-ch10] 10.5), or
 *    sigmoid affinities renormalised over the selected (DeepSeek-V3 style);
 *  - group limit: experts are split into G groups of consecutive indices, only
 *    the kg groups with the highest group score stay eligible (each token
 *    reaches experts on a bounded number of nodes, [EP-glossary] "Load
 *    balancing and capacity", last paragraph);
 *  - top-k: the k eligible experts with the highest selection scores
 *    ([EP-glossary] step 1 "keep the k highest-scoring experts");
 *  - weights: from the unbiased scores of the selected experts; the outputs
 *    are later weighted by them and summed ([EP-glossary] step 4). */
static void select_token(const oracle_desc* desc, const float* zt, const float* sel_bias,
                         int32_t* idx, float* wout, float* aff, float* s,
                         unsigned char* eligible, float* gscore, unsigned char* gkeep) {
  const int32_t E = desc->num_experts, k = desc->top_k;
  const int32_t G = desc->num_groups, kg = desc->topk_groups, per = E / G;

  for (int32_t e = 0; e < E; ++e) {
    const float a = desc->score_fn == 2 ? sigmoid_affinity(zt[e]) : zt[e];
    if (aff) aff[e] = a;
    s[e] = sel_bias ? a + sel_bias[e] : a; /* fp32 add */
    eligible[e] = 1;
  }

  if (G > 1) {
    for (int32_t g = 0; g < G; ++g) {
      float m = s[g * per];
      for (int32_t e = g * per + 1; e < (g + 1) * per; ++e)
        if (s[e] > m) m = s[e];
      gscore[g] = m;
      gkeep[g] = 0;
    }
    for (int32_t j = 0; j < kg; ++j) {
      int32_t best = -1;
      for (int32_t g = 0; g < G; ++g)
        if (!gkeep[g] && (best < 0 || ranks_before(gscore[g], g, gscore[best], best))) best = g;
      gkeep[best] = 1;
    }
    for (int32_t e = 0; e < E; ++e) eligible[e] = gkeep[e / per];
  }

  for (int32_t j = 0; j < k; ++j) {
    int32_t best = -1;
    for (int32_t e = 0; e < E; ++e)
      if (eligible[e] && (best < 0 || ranks_before(s[e], e, s[best], best))) best = e;
    idx[j] = best;
    eligible[best] = 0; /* taken */
  }

  if (desc->score_fn == 0) {
    double zmax = -INFINITY;
    for (int32_t j = 0; j < k; ++j) zmax = fmax(zmax, (double)zt[idx[j]]);
    double sum = 0.0;
    for (int32_t j = 0; j < k; ++j) sum += exp((double)zt[idx[j]] - zmax);
    for (int32_t j = 0; j < k; ++j) wout[j] = (float)(exp((double)zt[idx[j]] - zmax) / sum);
  } else if (desc->score_fn == 1) {
    double zmax = -INFINITY;
    for (int32_t e = 0; e < E; ++e) zmax = fmax(zmax, (double)zt[e]);
    double sum = 0.0;
    for (int32_t e = 0; e < E; ++e) sum += exp((double)zt[e] - zmax);
    for (int32_t j = 0; j < k; ++j) wout[j] = (float)(exp((double)zt[idx[j]] - zmax) / sum);
  } else {
    double sum = 0.0;
    for (int32_t j = 0; j < k; ++j) sum += (double)sigmoid_affinity(zt[idx[j]]);
    for (int32_t j = 0; j < k; ++j) wout[j] = (float)((double)sigmoid_affinity(zt[idx[j]]) / sum);
  }
}

int oracle_select(const oracle_desc* desc, const float* z, const float* sel_bias,
                  int32_t* topk_idx, float* topk_w, int32_t* counts, float* affinity) {
  if (!desc_ok(desc) || !counts || (desc->num_tokens > 0 && (!z || !topk_idx || !topk_w)))
    return -1;
  const int32_t N = desc->num_tokens, E = desc->num_experts, k = desc->top_k;
  const int32_t G = desc->num_groups;
  int failed = 0;
#pragma omp parallel num_threads(g_threads)
  {
    float* s = (float*)malloc(sizeof(float) * E);
    unsigned char* elig = (unsigned char*)malloc((size_t)E);
    float* gs = (float*)malloc(sizeof(float) * G);
    unsigned char* gk = (unsigned char*)malloc((size_t)G);
    if (!s || !elig || !gs || !gk) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(static)
    for (int32_t t = 0; t < N; ++t) {
      if (!s || !elig || !gs || !gk) continue;
      select_token(desc, z + (size_t)t * E, sel_bias, topk_idx + (size_t)t * k,
                   topk_w + (size_t)t * k, affinity ? affinity + (size_t)t * E : NULL, s, elig,
                   gs, gk);
    }
    free(s);
    free(elig);
    free(gs);
    free(gk);
  }
  if (failed) return -1;
  /* Per-expert assignment counts (the snippet's bincount over the chosen
   * experts, [EP-glossary] routing snippet). */
  for (int32_t e = 0; e < E; ++e) counts[e] = 0;
  for (size_t i = 0; i < (size_t)N * k; ++i) counts[topk_idx[i]] += 1;
  return 0;
}

/* -------------------------------------------------------------- dispatch -- */

/* Capacity: each expert takes at most a fixed number of token-expert
 * assignments per batch, the factor times its uniform share N*k/E
 * ([EP-glossary] "Load balancing and capacity", capacity-factor bullet;
 * [EP-notes] answer 2: per-expert buffer = mean x 1.25). */
int64_t oracle_capacity(const oracle_desc* desc) {
  if (!desc || desc->capacity_factor <= 0.0f) return INT32_MAX;
  double c = ceil((double)desc->capacity_factor * ((double)desc->num_tokens * desc->top_k) /
                  (double)desc->num_experts);
  return c > (double)INT32_MAX ? INT32_MAX : (int64_t)c;
}

/* Dispatch layout.  Tokens are taken in order; a slot whose expert is already
 * full is dropped (it "skips that expert").  Rows are grouped by expert, and
 * experts are placed on ranks in blocks, rank = e / (E/R) (the snippet's
 * `experts // (num_experts // num_gpus)`), so the same buffer is contiguous per
 * rank: it is the send buffer of the dispatch all-to-all and rank_counts are
 * its send counts ([EP-glossary] step 2; [EP-notes] dispatch). */
int oracle_dispatch(const oracle_desc* desc, const int32_t* topk_idx,
                    int32_t* row_of_slot, int32_t* token_of_row, int8_t* slot_of_row,
                    int32_t* expert_offsets, int32_t* admitted,
                    int32_t* rank_offsets, int32_t* rank_counts) {
  return oracle_dispatch_ex(desc, 0, topk_idx, row_of_slot, token_of_row, slot_of_row,
                            expert_offsets, admitted, rank_offsets, rank_counts);
}

int oracle_dispatch_ex(const oracle_desc* desc, int32_t admission, const int32_t* topk_idx,
                       int32_t* row_of_slot, int32_t* token_of_row, int8_t* slot_of_row,
                       int32_t* expert_offsets, int32_t* admitted,
                       int32_t* rank_offsets, int32_t* rank_counts) {
  if (!desc_ok(desc) || !expert_offsets || !admitted || !rank_offsets || !rank_counts) return -1;
  if (admission & ~3) return -1;
  const int first_choice = admission & 1, padded = (admission >> 1) & 1;
  const int32_t N = desc->num_tokens, E = desc->num_experts, k = desc->top_k;
  const int32_t R = desc->num_ranks;
  const size_t S = (size_t)N * k;
  if (S > 0 && (!topk_idx || !row_of_slot || !token_of_row || !slot_of_row)) return -1;
  for (size_t i = 0; i < S; ++i)
    if (topk_idx[i] < 0 || topk_idx[i] >= E) return -1;
  const int64_t cap = oracle_capacity(desc);
  /* The padded layout needs a finite capacity and E * cap rows. */
  if (padded && (desc->capacity_factor <= 0.0f || (int64_t)E * cap > INT32_MAX)) return -1;
  const size_t rows_total = padded && (size_t)E * (size_t)cap > S ? (size_t)E * (size_t)cap : S;

  int32_t* seen = (int32_t*)calloc((size_t)E, sizeof(int32_t));
  int32_t* rank_in_expert = (int32_t*)malloc(sizeof(int32_t) * (S ? S : 1));
  int32_t* counts = (int32_t*)calloc((size_t)E, sizeof(int32_t));
  if (!seen || !rank_in_expert || !counts) {
    free(seen);
    free(rank_in_expert);
    free(counts);
    return -1;
  }
  for (size_t i = 0; i < S; ++i) counts[topk_idx[i]] += 1;

  if (!first_choice) {
    /* Admission in token order (t outer, slot inner). */
    for (int32_t t = 0; t < N; ++t) {
      for (int32_t j = 0; j < k; ++j) {
        const size_t slot = (size_t)t * k + j;
        const int32_t e = topk_idx[slot];
        if (seen[e] < cap) {
          rank_in_expert[slot] = seen[e];
          seen[e] += 1;
        } else {
          rank_in_expert[slot] = -1; /* dropped */
        }
      }
    }
  } else {
    /* First choice first: every token's slot 0 (in token order), then every
     * token's slot 1, and so on (slot outer, token inner). */
    for (int32_t j = 0; j < k; ++j) {
      for (int32_t t = 0; t < N; ++t) {
        const size_t slot = (size_t)t * k + j;
        const int32_t e = topk_idx[slot];
        if (seen[e] < cap) {
          rank_in_expert[slot] = seen[e];
          seen[e] += 1;
        } else {
          rank_in_expert[slot] = -1; /* dropped */
        }
      }
    }
  }

  /* Compact layout: expert e's rows follow expert e-1's admitted rows.
   * Padded layout (GShard's fixed buffers of cap rows per expert): expert e
   * owns rows [e cap, (e+1) cap); the rows past its admitted ones are padding. */
  int32_t run = 0;
  for (int32_t e = 0; e < E; ++e) {
    admitted[e] = counts[e] < cap ? counts[e] : (int32_t)cap;
    expert_offsets[e] = padded ? (int32_t)(e * cap) : run;
    run += admitted[e];
  }
  expert_offsets[E] = padded ? (int32_t)(E * cap) : run;

  for (size_t i = 0; i < rows_total; ++i) {
    token_of_row[i] = -1;
    slot_of_row[i] = -1;
  }
  for (int32_t t = 0; t < N; ++t) {
    for (int32_t j = 0; j < k; ++j) {
      const size_t slot = (size_t)t * k + j;
      if (rank_in_expert[slot] < 0) {
        row_of_slot[slot] = -1;
        continue;
      }
      const int32_t row = expert_offsets[topk_idx[slot]] + rank_in_expert[slot];
      row_of_slot[slot] = row;
      token_of_row[row] = t;
      slot_of_row[row] = (int8_t)j;
    }
  }

  const int32_t per = E / R;
  for (int32_t r = 0; r <= R; ++r) rank_offsets[r] = expert_offsets[r * per];
  for (int32_t r = 0; r < R; ++r) rank_counts[r] = rank_offsets[r + 1] - rank_offsets[r];

  free(seen);
  free(rank_in_expert);
  free(counts);
  return 0;
}

/* The dispatch payload: each admitted row carries its token's hidden state
 * unchanged ([EP-glossary] step 2). */
int oracle_permute(int32_t num_rows, int32_t hidden, int32_t dtype, const void* x,
                   const int32_t* token_of_row, void* x_perm) {
  if (num_rows < 0 || hidden < 1 || !dtype_ok(dtype)) return -1;
  if (num_rows > 0 && (!x || !token_of_row || !x_perm)) return -1;
  const size_t es = dtype == 0 ? 4 : 2, rb = es * (size_t)hidden;
  for (int32_t i = 0; i < num_rows; ++i) {
    if (token_of_row[i] < 0) /* a padding row of the padded layout */
      memset((char*)x_perm + (size_t)i * rb, 0, rb);
    else
      memcpy((char*)x_perm + (size_t)i * rb, (const char*)x + (size_t)token_of_row[i] * rb, rb);
  }
  return 0;
}

/* ----------------------------------------------------- INT8 payload -- */

/* INT8 payload of the dispatch exchange (EP notes, "深入推导": INT8-quantised
 * communication halves the exchange volume).  The pages give no scheme; the
 * reading taken is one symmetric scale per token row, and every decision is an
 * fp32 IEEE operation rounded to nearest even:
 *   amax = max_i |x_i|  (exact);  amax == 0: q = 0, s = 0;  otherwise
 *   inv  = 127 / amax,  q_i = clamp(rint(x_i * inv), -127, 127),  s = amax / 127. */
int oracle_quantize_rows_q8(int32_t num_rows, int32_t hidden, int32_t dtype, const void* x,
                            int8_t* q, float* scale) {
  if (num_rows < 0 || hidden < 1 || !dtype_ok(dtype)) return -1;
  if (num_rows > 0 && (!x || !q || !scale)) return -1;
  for (int32_t r = 0; r < num_rows; ++r) {
    const size_t base = (size_t)r * hidden;
    float amax = 0.0f;
    for (int32_t i = 0; i < hidden; ++i) {
      const float v = fabsf((float)elem(x, dtype, base + i));
      if (v > amax) amax = v;
    }
    if (amax == 0.0f) {
      for (int32_t i = 0; i < hidden; ++i) q[base + i] = 0;
      scale[r] = 0.0f;
      continue;
    }
    const float inv = 127.0f / amax;
    for (int32_t i = 0; i < hidden; ++i) {
      const float v = (float)elem(x, dtype, base + i) * inv;
      float c = rintf(v);
      if (c > 127.0f) c = 127.0f;
      if (c < -127.0f) c = -127.0f;
      q[base + i] = (int8_t)c;
    }
    scale[r] = amax / 127.0f;
  }
  return 0;
}

/* x'_i = q_i * s as an fp32 product, then rounded to the dtype (bf16: nearest
 * even; fp32: unchanged). */
int oracle_dequantize_rows_q8(int32_t num_rows, int32_t hidden, int32_t dtype, const int8_t* q,
                              const float* scale, void* x) {
  if (num_rows < 0 || hidden < 1 || !dtype_ok(dtype)) return -1;
  if (num_rows > 0 && (!x || !q || !scale)) return -1;
  for (int32_t r = 0; r < num_rows; ++r) {
    for (int32_t i = 0; i < hidden; ++i) {
      const size_t k = (size_t)r * hidden + i;
      const float v = (float)q[k] * scale[r];
      if (dtype == 0)
        ((float*)x)[k] = v;
      else
        ((uint16_t*)x)[k] = double_to_bf16_bits((double)v);
    }
  }
  return 0;
}

/* ------------------------------------------------------------ expert FFN -- */

static double act_relu(double u) { return u > 0.0 ? u : 0.0; }
static double act_gelu(double u) { return 0.5 * u * (1.0 + erf(u / sqrt(2.0))); }
static double act_silu(double g) { return g / (1.0 + exp(-g)); }

/* Each expert is an ordinary feed-forward block ([EP-glossary] intro: the MoE
 * layer replaces one large feed-forward block by many small expert networks;
 * [EP-notes] "为何不用 TP 切专家": a single expert is an ordinary FFN).
 * H = act(x W1^T) (SwiGLU: silu(x W1^T) * (x W3^T)), rounded to the dtype;
 * y = H W2^T, rounded to the dtype.  Sums in fp64. */
int oracle_ffn_row(int32_t hidden, int32_t ffn_hidden, int32_t act, int32_t dtype,
                   const void* x_row, const void* w1, const void* w3, const void* w2,
                   void* y_row) {
  if (hidden < 1 || ffn_hidden < 1 || act < 0 || act > 2 || !dtype_ok(dtype)) return -1;
  if (!x_row || !w1 || !w2 || !y_row || (act == 2 && !w3)) return -1;
  const int32_t d = hidden, h = ffn_hidden;
  double* xd = (double*)malloc(sizeof(double) * d);
  double* hd = (double*)malloc(sizeof(double) * h);
  if (!xd || !hd) {
    free(xd);
    free(hd);
    return -1;
  }
  for (int32_t i = 0; i < d; ++i) xd[i] = elem(x_row, dtype, i);
  for (int32_t j = 0; j < h; ++j) {
    double u = 0.0;
    for (int32_t i = 0; i < d; ++i) u += xd[i] * elem(w1, dtype, (size_t)j * d + i);
    double a;
    if (act == 0) {
      a = act_relu(u);
    } else if (act == 1) {
      a = act_gelu(u);
    } else {
      double v = 0.0;
      for (int32_t i = 0; i < d; ++i) v += xd[i] * elem(w3, dtype, (size_t)j * d + i);
      a = act_silu(u) * v;
    }
    /* H is stored in the layer dtype before the second projection. */
    hd[j] = dtype == 0 ? (double)(float)a : bf16_bits_to_double(double_to_bf16_bits(a));
  }
  for (int32_t i = 0; i < d; ++i) {
    double o = 0.0;
    for (int32_t j = 0; j < h; ++j) o += hd[j] * elem(w2, dtype, (size_t)i * h + j);
    store(y_row, dtype, (size_t)i, o);
  }
  free(xd);
  free(hd);
  return 0;
}

int oracle_expert_ffn(int32_t num_experts, int32_t hidden, int32_t ffn_hidden,
                      int32_t act, int32_t dtype, const void* x_rows,
                      const int32_t* offsets, const void* w1, const void* w3,
                      const void* w2, void* y_rows) {
  if (num_experts < 1 || hidden < 1 || ffn_hidden < 1 || !dtype_ok(dtype) || !offsets)
    return -1;
  if (act < 0 || act > 2) return -1;
  const size_t es = dtype == 0 ? 4 : 2;
  const size_t wsz = (size_t)hidden * ffn_hidden * es;
  const size_t rb = (size_t)hidden * es;
  for (int32_t e = 0; e < num_experts; ++e)
    if (offsets[e + 1] < offsets[e] || offsets[e] < 0) return -1;
  int failed = 0;
  for (int32_t e = 0; e < num_experts; ++e) {
    const int32_t lo = offsets[e], hi = offsets[e + 1];
    const char* w1e = (const char*)w1 + (size_t)e * wsz;
    const char* w3e = w3 ? (const char*)w3 + (size_t)e * wsz : NULL;
    const char* w2e = (const char*)w2 + (size_t)e * wsz;
#pragma omp parallel for num_threads(g_threads) schedule(dynamic, 1)
    for (int32_t r = lo; r < hi; ++r) {
      if (oracle_ffn_row(hidden, ffn_hidden, act, dtype, (const char*)x_rows + (size_t)r * rb,
                         w1e, w3e, w2e, (char*)y_rows + (size_t)r * rb) != 0) {
#pragma omp atomic write
        failed = 1;
      }
    }
  }
  return failed ? -1 : 0;
}

/* --------------------------------------------------- expert FFN backward -- */

/* Derivatives of the activations (the gradients of the layer's expert
 * networks, the backward of the layer).  gelu(u) = u Phi(u), so
 * gelu'(u) = Phi(u) + u phi(u); silu(u) = u s(u) with s the logistic
 * function, so silu'(u) = s(u) (1 + u (1 - s(u))). */
static double dact_relu(double u) { return u > 0.0 ? 1.0 : 0.0; }
static double dact_gelu(double u) {
  const double pi = 3.14159265358979323846;
  return 0.5 * (1.0 + erf(u / sqrt(2.0))) + u * exp(-0.5 * u * u) / sqrt(2.0 * pi);
}
static double dact_silu(double u) {
  const double s = 1.0 / (1.0 + exp(-u));
  return s * (1.0 + u * (1.0 - s));
}
static double round_dt(int32_t dtype, double v) {
  return dtype == 0 ? (double)(float)v : bf16_bits_to_double(double_to_bf16_bits(v));
}

/* One row through the backward of one expert, by the chain rule through the
 * forward of oracle_ffn_row (u = x W1^T, v = x W3^T, H = act(u) [* v],
 * y = H W2^T):
 *   g  = dy W2                 (gradient at H; fp64 sums)
 *   du = g * act'(u) [* v]     (gradient at u), rounded to the dtype
 *   dv = g * silu(u)           (SwiGLU: gradient at v), rounded to the dtype
 *   dx = du W1 [+ dv W3]       (fp64 sums), rounded to the dtype.
 * h_out, du_out and dv_out (nullable) receive H (rounded as in the forward),
 * du and dv: the operands of the weight gradients. */
int oracle_ffn_backward_row(int32_t hidden, int32_t ffn_hidden, int32_t act, int32_t dtype,
                            const void* x_row, const void* w1, const void* w3, const void* w2,
                            const void* dy_row, void* dx_row, double* h_out, double* du_out,
                            double* dv_out) {
  if (hidden < 1 || ffn_hidden < 1 || act < 0 || act > 2 || !dtype_ok(dtype)) return -1;
  if (!x_row || !w1 || !w2 || !dy_row || !dx_row || (act == 2 && !w3)) return -1;
  const int32_t d = hidden, h = ffn_hidden;
  double* xd = (double*)malloc(sizeof(double) * d);
  double* dyd = (double*)malloc(sizeof(double) * d);
  double* du = (double*)malloc(sizeof(double) * h);
  double* dv = (double*)malloc(sizeof(double) * h);
  if (!xd || !dyd || !du || !dv) {
    free(xd);
    free(dyd);
    free(du);
    free(dv);
    return -1;
  }
  for (int32_t i = 0; i < d; ++i) {
    xd[i] = elem(x_row, dtype, i);
    dyd[i] = elem(dy_row, dtype, i);
  }
  for (int32_t j = 0; j < h; ++j) {
    double u = 0.0, v = 0.0, g = 0.0;
    for (int32_t i = 0; i < d; ++i) u += xd[i] * elem(w1, dtype, (size_t)j * d + i);
    if (act == 2)
      for (int32_t i = 0; i < d; ++i) v += xd[i] * elem(w3, dtype, (size_t)j * d + i);
    for (int32_t i = 0; i < d; ++i) g += dyd[i] * elem(w2, dtype, (size_t)i * h + j);
    double hv, dgu, dgv = 0.0;
    if (act == 0) {
      hv = act_relu(u);
      dgu = g * dact_relu(u);
    } else if (act == 1) {
      hv = act_gelu(u);
      dgu = g * dact_gelu(u);
    } else {
      hv = act_silu(u) * v;
      dgu = g * dact_silu(u) * v;
      dgv = g * act_silu(u);
    }
    du[j] = round_dt(dtype, dgu);
    dv[j] = round_dt(dtype, dgv);
    if (h_out) h_out[j] = round_dt(dtype, hv);
    if (du_out) du_out[j] = du[j];
    if (dv_out) dv_out[j] = dv[j];
  }
  for (int32_t i = 0; i < d; ++i) {
    double o = 0.0;
    for (int32_t j = 0; j < h; ++j) o += du[j] * elem(w1, dtype, (size_t)j * d + i);
    if (act == 2)
      for (int32_t j = 0; j < h; ++j) o += dv[j] * elem(w3, dtype, (size_t)j * d + i);
    store(dx_row, dtype, (size_t)i, o);
  }
  free(xd);
  free(dyd);
  free(du);
  free(dv);
  return 0;
}

/* Backward of the grouped FFN: rows [offsets[e], offsets[e+1]) of x_rows and
 * dy_rows belong to expert e.  dx_rows gets every such row's input gradient;
 * the weight gradients sum over the expert's rows (fp64 sums, stored fp32):
 *   dw1[e][j][i] = sum_r du[r][j] x[r][i],  dw3[e][j][i] = sum_r dv[r][j] x[r][i],
 *   dw2[e][i][j] = sum_r dy[r][i] H[r][j].
 * An expert with no rows gets zero weight gradients; dw3 only for SwiGLU. */
int oracle_expert_ffn_backward(int32_t num_experts, int32_t hidden, int32_t ffn_hidden,
                               int32_t act, int32_t dtype, const void* x_rows,
                               const int32_t* offsets, const void* w1, const void* w3,
                               const void* w2, const void* dy_rows, void* dx_rows, float* dw1,
                               float* dw3, float* dw2) {
  if (num_experts < 1 || hidden < 1 || ffn_hidden < 1 || !dtype_ok(dtype) || !offsets)
    return -1;
  if (act < 0 || act > 2 || !dw1 || !dw2 || (act == 2 && (!w3 || !dw3))) return -1;
  const int32_t d = hidden, h = ffn_hidden;
  const size_t es = dtype == 0 ? 4 : 2;
  const size_t wsz = (size_t)d * h * es, rb = (size_t)d * es;
  for (int32_t e = 0; e < num_experts; ++e)
    if (offsets[e + 1] < offsets[e] || offsets[e] < 0) return -1;
  int failed = 0;
  for (int32_t e = 0; e < num_experts && !failed; ++e) {
    const int32_t lo = offsets[e], n = offsets[e + 1] - offsets[e];
    const char* w1e = (const char*)w1 + (size_t)e * wsz;
    const char* w3e = w3 ? (const char*)w3 + (size_t)e * wsz : NULL;
    const char* w2e = (const char*)w2 + (size_t)e * wsz;
    float* g1 = dw1 + (size_t)e * h * d;
    float* g3 = act == 2 ? dw3 + (size_t)e * h * d : NULL;
    float* g2 = dw2 + (size_t)e * d * h;
    const size_t cells = (size_t)(n > 0 ? n : 1) * h;
    double* H = (double*)malloc(sizeof(double) * cells);
    double* du = (double*)malloc(sizeof(double) * cells);
    double* dv = (double*)malloc(sizeof(double) * cells);
    if (!H || !du || !dv) {
      free(H);
      free(du);
      free(dv);
      return -1;
    }
#pragma omp parallel for num_threads(g_threads) schedule(dynamic, 1)
    for (int32_t r = 0; r < n; ++r) {
      if (oracle_ffn_backward_row(d, h, act, dtype, (const char*)x_rows + (size_t)(lo + r) * rb,
                                  w1e, w3e, w2e, (const char*)dy_rows + (size_t)(lo + r) * rb,
                                  (char*)dx_rows + (size_t)(lo + r) * rb, H + (size_t)r * h,
                                  du + (size_t)r * h, dv + (size_t)r * h) != 0) {
#pragma omp atomic write
        failed = 1;
      }
    }
#pragma omp parallel for num_threads(g_threads) schedule(static)
    for (int32_t j = 0; j < h; ++j) {
      for (int32_t i = 0; i < d; ++i) {
        double s1 = 0.0, s3 = 0.0;
        for (int32_t r = 0; r < n; ++r) {
          const double xv = elem(x_rows, dtype, (size_t)(lo + r) * d + i);
          s1 += du[(size_t)r * h + j] * xv;
          s3 += dv[(size_t)r * h + j] * xv;
        }
        g1[(size_t)j * d + i] = (float)s1;
        if (g3) g3[(size_t)j * d + i] = (float)s3;
      }
    }
#pragma omp parallel for num_threads(g_threads) schedule(static)
    for (int32_t i = 0; i < d; ++i) {
      for (int32_t j = 0; j < h; ++j) {
        double s2 = 0.0;
        for (int32_t r = 0; r < n; ++r)
          s2 += elem(dy_rows, dtype, (size_t)(lo + r) * d + i) * H[(size_t)r * h + j];
        g2[(size_t)i * h + j] = (float)s2;
      }
    }
    free(H);
    free(du);
    free(dv);
  }
  return failed ? -1 : 0;
}

/* --------------------------------------------------------------- combine -- */

/* Combine: each token's expert outputs come back to it, weighted by the router
 * scores and summed ([EP-glossary] step 4; [EP-notes] combine).  The layer
 * output carries the residual, so a token whose every slot was dropped leaves
 * the layer unchanged ([EP-glossary] "Load balancing and capacity", the
 * paragraph after the capacity list).  A DeepSeek-style shared expert output
 * is added with weight 1.  One rounding to the dtype at the end. */
int oracle_combine(int32_t num_tokens, int32_t hidden, int32_t top_k, int32_t dtype,
                   const void* y_perm, const int32_t* row_of_slot, const float* topk_w,
                   const void* residual, const void* shared_out, void* y) {
  if (num_tokens < 0 || hidden < 1 || top_k < 1 || !dtype_ok(dtype)) return -1;
  if (num_tokens > 0 && (!row_of_slot || !topk_w || !y)) return -1;
  for (int32_t t = 0; t < num_tokens; ++t) {
    for (int32_t i = 0; i < hidden; ++i) {
      const size_t ti = (size_t)t * hidden + i;
      double acc = residual ? elem(residual, dtype, ti) : 0.0;
      if (shared_out) acc += elem(shared_out, dtype, ti);
      for (int32_t j = 0; j < top_k; ++j) {
        const int32_t row = row_of_slot[(size_t)t * top_k + j];
        if (row < 0) continue;
        if (!y_perm) return -1;
        acc += (double)topk_w[(size_t)t * top_k + j] *
               elem(y_perm, dtype, (size_t)row * hidden + i);
      }
      store(y, dtype, ti, acc);
    }
  }
  return 0;
}

/* Backward of the combine's expert terms (the layer's training step reads the
 * four steps of [EP-glossary] "How tokens travel between GPUs" backwards): for
 * every admitted slot (t, j) with row r = row_of_slot[t, j] and weight w,
 *   dy_perm[r]    = w * dy[t]                    (fp64, rounded once to the dtype)
 *   dtopk_w[t, j] = sum_i dy[t, i] * y_perm[r, i] (fp64, rounded once to fp32)
 * A dropped slot gets dtopk_w = 0 and writes no row.  The residual and shared
 * terms pass dy through unchanged (no computation).  The permute's backward is
 * the combine itself with unit weights and no residual: dx[t] = sum over the
 * token's admitted rows of dx_perm (oracle_combine). */
int oracle_combine_backward(int32_t num_tokens, int32_t hidden, int32_t top_k, int32_t dtype,
                            const void* dy, const void* y_perm, const int32_t* row_of_slot,
                            const float* topk_w, void* dy_perm, float* dtopk_w) {
  if (num_tokens < 0 || hidden < 1 || top_k < 1 || !dtype_ok(dtype)) return -1;
  if (num_tokens > 0 && (!dy || !y_perm || !row_of_slot || !topk_w || !dy_perm || !dtopk_w))
    return -1;
  for (int32_t t = 0; t < num_tokens; ++t) {
    for (int32_t j = 0; j < top_k; ++j) {
      const size_t slot = (size_t)t * top_k + j;
      const int32_t row = row_of_slot[slot];
      if (row < 0) {
        dtopk_w[slot] = 0.0f;
        continue;
      }
      const double w = (double)topk_w[slot];
      double dot = 0.0;
      for (int32_t i = 0; i < hidden; ++i) {
        const double g = elem(dy, dtype, (size_t)t * hidden + i);
        dot += g * elem(y_perm, dtype, (size_t)row * hidden + i);
        store(dy_perm, dtype, (size_t)row * hidden + i, w * g);
      }
      dtopk_w[slot] = (float)dot;
    }
  }
  return 0;
}

/* ------------------------------------------------------- router backward -- */

/* Backward of the router (the training step reads step 1 of [EP-glossary] "How
 * tokens travel between GPUs" backwards) plus an auxiliary load-balancing loss
 * ([EP-glossary] "Load balancing and capacity", auxiliary-loss bullet; [MLSys
 * ch.10] 10.5 names it for GShard; the pages give no formula).
 *
 * Given the router logits z [N,E], the selection topk_idx [N,k] and the
 * gradient dtopk_w [N,k] of the loss at the combine weights, per token:
 *  - softmax over the k selected (score_fn 0): w_j = e^{z_j} / sum_sel e^{z};
 *    dz at selected expert e_j = w_j (g_j - sum_i w_i g_i), 0 elsewhere;
 *  - softmax over all E (score_fn 1): p = softmax(z), w_j = p_{e_j};
 *    dz_e = p_e (G_e - sum_j p_{e_j} g_j), G_e = g_j if e = e_j else 0;
 *  - sigmoid renormalised (score_fn 2): a = 1/(1+e^{-z}), S = sum_sel a,
 *    w_j = a_j / S; dz at e_j = a_j (1 - a_j) (g_j - sum_i w_i g_i) / S.
 * The selection (top-k, group limit, selection bias) is piecewise constant in
 * z: it passes no gradient.  Dropped slots arrive with g = 0.
 *
 * Auxiliary loss (reading: the load-balancing loss of the Switch Transformer,
 * generalised to k slots): L = coef * E * sum_e f_e P_e with f_e = counts_e /
 * (N k) (the fraction of assignments routed to e, a constant) and P_e the mean
 * over tokens of the token's router distribution: softmax(z) for the softmax
 * score functions, a_e / sum_all a for the sigmoid one.  Its gradient adds
 *   coef E / N * P_e' (f_e' - sum_e f_e P_e)                 (softmax)
 *   coef E / N * a_e'(1 - a_e') (f_e' - sum_e f_e P_e) / A   (sigmoid, A = sum a)
 * to dz[t, e'].  coef = 0: no auxiliary loss (aux_loss = 0).
 *
 * Through the router z = x W_r^T + b:  dW_r[e] = sum_t dz[t,e] x[t],
 * db[e] = sum_t dz[t,e], dx[t] = sum_e dz[t,e] W_r[e] (plus dx_in[t] when
 * given: the rest of the layer's input gradient, so one rounding covers both).
 * Everything in fp64; dz, dW_r, db rounded once to fp32, dx to the dtype. */
int oracle_router_backward(const oracle_desc* desc, const void* x, const void* w_router,
                           const float* z, const int32_t* topk_idx, const float* dtopk_w,
                           const int32_t* counts, double aux_coef, const void* dx_in,
                           float* dz_out, float* dw_router, float* db, void* dx,
                           double* aux_loss) {
  if (!desc_ok(desc) || !dz_out || !dw_router || !aux_loss) return -1;
  const int32_t N = desc->num_tokens, d = desc->hidden, E = desc->num_experts;
  const int32_t k = desc->top_k, sf = desc->score_fn;
  if (N > 0 && (!x || !w_router || !z || !topk_idx || !dtopk_w || !dx)) return -1;
  if (aux_coef != 0.0 && !counts) return -1;
  for (size_t i = 0; i < (size_t)N * k; ++i)
    if (topk_idx[i] < 0 || topk_idx[i] >= E) return -1;
  double* dz = (double*)calloc((size_t)N * E + 1, sizeof(double));
  double* pbar = (double*)calloc((size_t)E + 1, sizeof(double));
  double* f = (double*)calloc((size_t)E + 1, sizeof(double));
  double* p = (double*)malloc(sizeof(double) * ((size_t)E + 1));
  double* w = (double*)malloc(sizeof(double) * ((size_t)k + 1));
  if (!dz || !pbar || !f || !p || !w) {
    free(dz); free(pbar); free(f); free(p); free(w);
    return -1;
  }
  if (aux_coef != 0.0 && N > 0)
    for (int32_t e = 0; e < E; ++e) f[e] = (double)counts[e] / ((double)N * k);

  for (int32_t t = 0; t < N; ++t) {
    const float* zt = z + (size_t)t * E;
    const int32_t* idx = topk_idx + (size_t)t * k;
    const float* g = dtopk_w + (size_t)t * k;
    double* dzt = dz + (size_t)t * E;
    /* the token's router distribution over all E (aux loss; softmax-all weights) */
    double A = 0.0;
    if (sf == 2) {
      for (int32_t e = 0; e < E; ++e) {
        p[e] = 1.0 / (1.0 + exp(-(double)zt[e]));
        A += p[e];
      }
    } else {
      double zmax = -INFINITY;
      for (int32_t e = 0; e < E; ++e) zmax = fmax(zmax, (double)zt[e]);
      for (int32_t e = 0; e < E; ++e) {
        p[e] = exp((double)zt[e] - zmax);
        A += p[e];
      }
      for (int32_t e = 0; e < E; ++e) p[e] /= A;
    }
    /* weights part */
    if (sf == 0) {
      double zmax = -INFINITY, sum = 0.0, wg = 0.0;
      for (int32_t j = 0; j < k; ++j) zmax = fmax(zmax, (double)zt[idx[j]]);
      for (int32_t j = 0; j < k; ++j) sum += exp((double)zt[idx[j]] - zmax);
      for (int32_t j = 0; j < k; ++j) {
        w[j] = exp((double)zt[idx[j]] - zmax) / sum;
        wg += w[j] * (double)g[j];
      }
      for (int32_t j = 0; j < k; ++j) dzt[idx[j]] += w[j] * ((double)g[j] - wg);
    } else if (sf == 1) {
      double pg = 0.0;
      for (int32_t j = 0; j < k; ++j) pg += p[idx[j]] * (double)g[j];
      for (int32_t e = 0; e < E; ++e) dzt[e] += -p[e] * pg;
      for (int32_t j = 0; j < k; ++j) dzt[idx[j]] += p[idx[j]] * (double)g[j];
    } else {
      double S = 0.0, wg = 0.0;
      for (int32_t j = 0; j < k; ++j) S += p[idx[j]];
      for (int32_t j = 0; j < k; ++j) wg += p[idx[j]] / S * (double)g[j];
      for (int32_t j = 0; j < k; ++j) {
        const double a = p[idx[j]];
        dzt[idx[j]] += a * (1.0 - a) * ((double)g[j] - wg) / S;
      }
    }
    /* auxiliary loss part */
    if (aux_coef != 0.0) {
      double fp = 0.0;
      const double scale = aux_coef * (double)E / (double)N;
      if (sf == 2) {
        for (int32_t e = 0; e < E; ++e) fp += f[e] * p[e] / A;
        for (int32_t e = 0; e < E; ++e) {
          pbar[e] += p[e] / A;
          dzt[e] += scale * p[e] * (1.0 - p[e]) * (f[e] - fp) / A;
        }
      } else {
        for (int32_t e = 0; e < E; ++e) fp += f[e] * p[e];
        for (int32_t e = 0; e < E; ++e) {
          pbar[e] += p[e];
          dzt[e] += scale * p[e] * (f[e] - fp);
        }
      }
    }
  }
  double loss = 0.0;
  if (aux_coef != 0.0 && N > 0)
    for (int32_t e = 0; e < E; ++e) loss += f[e] * (pbar[e] / (double)N);
  *aux_loss = aux_coef * (double)E * loss;

  for (size_t i = 0; i < (size_t)N * E; ++i) dz_out[i] = (float)dz[i];
  /* dW_r and db: sums over tokens in order */
  for (int32_t e = 0; e < E; ++e) {
    double be = 0.0;
    for (int32_t t = 0; t < N; ++t) be += dz[(size_t)t * E + e];
    if (db) db[e] = (float)be;
  }
#pragma omp parallel for num_threads(g_threads) schedule(static)
  for (int32_t e = 0; e < E; ++e) {
    for (int32_t i = 0; i < d; ++i) {
      double acc = 0.0;
      for (int32_t t = 0; t < N; ++t)
        acc += dz[(size_t)t * E + e] * elem(x, desc->dtype, (size_t)t * d + i);
      dw_router[(size_t)e * d + i] = (float)acc;
    }
  }
#pragma omp parallel for num_threads(g_threads) schedule(static)
  for (int32_t t = 0; t < N; ++t) {
    for (int32_t i = 0; i < d; ++i) {
      double acc = dx_in ? elem(dx_in, desc->dtype, (size_t)t * d + i) : 0.0;
      for (int32_t e = 0; e < E; ++e)
        acc += dz[(size_t)t * E + e] * elem(w_router, desc->dtype, (size_t)e * d + i);
      store(dx, desc->dtype, (size_t)t * d + i, acc);
    }
  }
  free(dz); free(pbar); free(f); free(p); free(w);
  return 0;
}

/* ------------------------------------------------------------ bias update -- */

/* Bias-based balancing: after each step the bias of overloaded experts goes
 * down and that of idle experts goes up ([EP-glossary] "Load balancing and
 * capacity", bias-based balancing bullet).  Load = pre-capacity assignment
 * count, compared with the mean N*k/E in integers (count*E vs N*k); equal
 * load leaves the bias as it is.  The step is applied in fp32. */
int oracle_bias_update(int32_t num_experts, int32_t num_tokens, int32_t top_k,
                       const int32_t* counts, float step, float* sel_bias) {
  if (num_experts < 1 || num_tokens < 0 || top_k < 1 || !counts || !sel_bias) return -1;
  const int64_t mean_times_e = (int64_t)num_tokens * top_k;
  for (int32_t e = 0; e < num_experts; ++e) {
    const int64_t load_times_e = (int64_t)counts[e] * num_experts;
    if (load_times_e > mean_times_e)
      sel_bias[e] = sel_bias[e] - step;
    else if (load_times_e < mean_times_e)
      sel_bias[e] = sel_bias[e] + step;
  }
  return 0;
}
