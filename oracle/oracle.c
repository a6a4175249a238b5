/*
 * oracle.c -- plain fp64 CPU reference for single-token grouped-query decode
 * attention over a paged, fp8-quantized KV cache, with an optional split-K
 * (flash-decoding) form and its log-sum-exp merge.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the library's product path may link,
 * load or call this file: only the tests, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header, table or helper with
 * the HIP path.
 *
 * What is computed (page "vllm.v1.attention.ops.flydsl_kernels.tq_decode",
 * docstring of build_tq_decode_module and STEPs B-G of tq_decode_kernel): for
 * every sequence s, kv head h and query row g of that head's group, the
 * attention of the single decode query against the sequence's first L_s
 * cached tokens, where token t lives in physical cache block
 * block_tables[s][t / BS] at slot t % BS (STEP F, block-table walk).
 *
 *   x_t   = softmax_scale * sum_d q[s][h*QG+g][d] * k_t[d]
 *   out   = sum_t exp(x_t - max x) v_t / sum_t exp(x_t - max x)
 *
 * Cache format (the pages leave the "TQ" contents open; this library fixes
 * fp8): K and V are OCP e4m3fn codes, one D-byte row per (block, kv head,
 * slot), each row carrying one fp32 scale for K and one for V, stored as SoA
 * metadata per cache block: kv_scales[NB][Hkv][2][BS] (field 0 = K, field 1 =
 * V), the kv_head-major order of the page's per-block metadata region (kv
 * head, then field, then slot).  The rows of a block are in one of two orders
 * (`layout`, see orc_row): head-major k_cache/v_cache[NB][Hkv][BS][D], or
 * slot-major [NB][BS][Hkv][D], the order of the page's data region.
 * Dequantized k_t[d] = e4m3fn(code) * scale.
 *
 * Everything is fp64: bf16 q and fp8 codes decode exactly, the fp32 scales and
 * the fp32 softmax_scale are widened, and exp() is libm's double exp().
 *
 * Second cache format, the page's 4-bit "TQ" record (STEP F: K dequantized as
 * centroids[index] * K norm, V as index * V scale + V zero point, the query
 * already rotated by the caller), in the reading this library takes where the
 * page leaves the constants open.  Cache block b is block_bytes =
 * Hkv*BS*D + Hkv*3*BS*2 bytes:
 *   data region  [Hkv][BS][D] (head-major) or [BS][Hkv][D] (slot-major, the
 *                page's order) bytes: the (head, slot) row holds the K indices
 *                in bytes 0..D/2-1 and the V indices in bytes D/2..D-1; dim d
 *                is byte d/2, low nibble for even d, high nibble for odd d
 *                (the page's word w, nibble n order, little-endian words);
 *   meta region  [Hkv][3][BS] IEEE fp16: field 0 = K norm, 1 = V scale,
 *                2 = V zero point;
 *   k_t[d] = centroids[kidx] * knorm,  v_t[d] = vidx * vscale + vzero,
 * with 16 fp32 centroids given by the caller.  The attention itself is the
 * one above.
 *
 * Split-K form (STEP E/F partition base and trip count, STEP G partial
 * stores): partition p of extent E tokens covers [p*E, min((p+1)*E, L)) and
 * yields m_p = max x, l_p = sum exp(x - m_p), o_p = sum exp(x - m_p) v / l_p
 * (the partial output normalised by its own sum, the max in natural-log units
 * of the scaled logits).  The merge -- not shown on the page; the reading used
 * here is the standard log-sum-exp merge of those three quantities -- is
 *   M = max_p m_p, w_p = l_p exp(m_p - M), out = sum_p w_p o_p / sum_p w_p
 * over live partitions only (p*E < L).  L = 0 gives 0.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_ERR_ARGS 1
#define ORC_ERR_BLOCK 2 /* a block-table entry needed for t < L is outside [0, NB) */
#define ORC_ERR_NOMEM 3

/* Order of the 128-byte K / V rows inside a cache block (the scale / metadata
 * region is [Hkv][field][BS] in both):
 *   head-major: row (h, slot) is row h * BS + slot   -- [BS rows of head 0][head 1]...
 *   slot-major: row (h, slot) is row slot * Hkv + h  -- the page's data region:
 *     STEP F addresses it as slot * _stride_data_slot + kv_h * DATA_BYTES_PER_SLOT,
 *     with _stride_data_slot = num_kv_heads * DATA_BYTES_PER_SLOT
 *     (build_tq_decode_module, "Strides"). */
#define ORC_LAYOUT_HEAD_MAJOR 0
#define ORC_LAYOUT_SLOT_MAJOR 1

/* Index of the row of (block blk, kv head h, slot) among the cache's rows. */
static int64_t orc_row(int32_t layout, int32_t Hkv, int32_t BS, int64_t blk, int h, int slot) {
  if (layout == ORC_LAYOUT_SLOT_MAJOR) return (blk * BS + slot) * Hkv + h;
  return (blk * Hkv + h) * BS + slot;
}

/* OCP 8-bit floating point, E4M3 variant "fn": 1 sign, 4 exponent bits (bias
 * 7), 3 mantissa bits, no infinities, S.1111.111 is NaN, largest finite 448. */
double orc_dec_e4m3fn(uint8_t code) {
  int sign = code >> 7;
  int e = (code >> 3) & 0xF;
  int m = code & 7;
  double mag;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    mag = ldexp((double)m, -9); /* subnormal: m/8 * 2^(1-7) */
  else
    mag = ldexp((double)(8 + m), e - 10); /* (1 + m/8) * 2^(e-7) */
  return sign ? -mag : mag;
}

/* bfloat16 is the high half of an IEEE binary32. */
double orc_dec_bf16(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* IEEE binary16: 1 sign, 5 exponent bits (bias 15), 10 mantissa bits. */
double orc_dec_f16(uint16_t bits) {
  int sign = bits >> 15;
  int e = (bits >> 10) & 0x1F;
  int m = bits & 0x3FF;
  double mag;
  if (e == 31) return m ? NAN : (sign ? -INFINITY : INFINITY);
  if (e == 0)
    mag = ldexp((double)m, -24); /* subnormal: m/1024 * 2^(1-15) */
  else
    mag = ldexp((double)(1024 + m), e - 25); /* (1 + m/1024) * 2^(e-15) */
  return sign ? -mag : mag;
}

typedef struct {
  const uint16_t* q;
  const uint8_t* k_cache;
  const uint8_t* v_cache;
  const float* kv_scales;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  int32_t S, Hkv, QG, D, BS, NB, max_blocks_per_seq;
  double scale;
  int32_t layout; /* ORC_LAYOUT_HEAD_MAJOR or ORC_LAYOUT_SLOT_MAJOR: order of a block's rows */
  /* 4-bit record format when tq4_cache is set (k_cache, v_cache, kv_scales unused) */
  const uint8_t* tq4_cache;
  const float* centroids;
} orc_problem;

/* Bytes of one 4-bit cache block. */
static int64_t orc_tq4_block_bytes(const orc_problem* pb) {
  return (int64_t)pb->Hkv * pb->BS * pb->D + (int64_t)pb->Hkv * 3 * pb->BS * 2;
}

/* Dequantized element d of the K (field 0) or V (field 1) row of (blk, h, slot)
 * in the 4-bit record format. */
static double orc_tq4_kv(const orc_problem* pb, int field, int blk, int slot, int h, int d) {
  const uint8_t* block = pb->tq4_cache + (int64_t)blk * orc_tq4_block_bytes(pb);
  const uint8_t* row = block + orc_row(pb->layout, pb->Hkv, pb->BS, 0, h, slot) * pb->D;
  const uint8_t* meta = block + (int64_t)pb->Hkv * pb->BS * pb->D + (int64_t)h * 3 * pb->BS * 2;
  int byte = row[(field == 0 ? 0 : pb->D / 2) + d / 2];
  int idx = (d & 1) ? byte >> 4 : byte & 0xF;
  uint16_t f[3];
  for (int i = 0; i < 3; ++i) memcpy(&f[i], meta + ((int64_t)i * pb->BS + slot) * 2, 2);
  if (field == 0) return (double)pb->centroids[idx] * orc_dec_f16(f[0]);
  return (double)idx * orc_dec_f16(f[1]) + orc_dec_f16(f[2]);
}

/* Physical block of token t of sequence s (STEP F block-table walk). */
static int orc_block(const orc_problem* pb, int s, int t, int* blk) {
  int32_t b = pb->block_tables[(int64_t)s * pb->max_blocks_per_seq + t / pb->BS];
  if (b < 0 || b >= pb->NB) return ORC_ERR_BLOCK;
  *blk = b;
  return ORC_OK;
}

/* Dequantized element d of the K (field 0) or V (field 1) row of token t. */
static double orc_kv(const orc_problem* pb, int field, int blk, int slot, int h, int d) {
  if (pb->tq4_cache) return orc_tq4_kv(pb, field, blk, slot, h, d);
  const uint8_t* cache = field == 0 ? pb->k_cache : pb->v_cache;
  int64_t row = orc_row(pb->layout, pb->Hkv, pb->BS, blk, h, slot);
  double code = orc_dec_e4m3fn(cache[row * pb->D + d]);
  double sc = (double)pb->kv_scales[(((int64_t)blk * pb->Hkv + h) * 2 + field) * pb->BS + slot];
  return code * sc;
}

/* Scaled logit x_t for query row (s, h, g). */
static int orc_logit(const orc_problem* pb, int s, int h, int g, int t, double* x) {
  int blk, rc = orc_block(pb, s, t, &blk);
  if (rc) return rc;
  const uint16_t* qrow = pb->q + ((int64_t)s * pb->Hkv * pb->QG + (int64_t)h * pb->QG + g) * pb->D;
  double dot = 0.0;
  for (int d = 0; d < pb->D; ++d) dot += orc_dec_bf16(qrow[d]) * orc_kv(pb, 0, blk, t % pb->BS, h, d);
  *x = pb->scale * dot;
  return ORC_OK;
}

/* Softmax-weighted V over tokens [t0, t1) of query row (s, h, g):
 * m = max x, l = sum exp(x - m), o[d] = sum exp(x - m) v[d] / l.
 * xbuf holds t1 - t0 doubles.  Requires t1 > t0. */
static int orc_attend(const orc_problem* pb, int s, int h, int g, int t0, int t1, double* xbuf,
                      double* o, double* m_out, double* l_out) {
  int rc;
  double m = -INFINITY, l = 0.0;
  for (int t = t0; t < t1; ++t) {
    rc = orc_logit(pb, s, h, g, t, &xbuf[t - t0]);
    if (rc) return rc;
    if (xbuf[t - t0] > m) m = xbuf[t - t0];
  }
  for (int d = 0; d < pb->D; ++d) o[d] = 0.0;
  for (int t = t0; t < t1; ++t) {
    int blk;
    double w = exp(xbuf[t - t0] - m);
    rc = orc_block(pb, s, t, &blk);
    if (rc) return rc;
    l += w;
    for (int d = 0; d < pb->D; ++d) o[d] += w * orc_kv(pb, 1, blk, t % pb->BS, h, d);
  }
  for (int d = 0; d < pb->D; ++d) o[d] /= l;
  *m_out = m;
  *l_out = l;
  return ORC_OK;
}

typedef struct {
  const orc_problem* pb;
  const int32_t* units; /* (s, h) pairs, or NULL for all S*Hkv in order */
  int32_t n_units;
  double* out; /* [n_units][QG][D] */
  int32_t next;
  int32_t rc;
  pthread_mutex_t lock;
} orc_job;

static void* orc_worker(void* arg) {
  orc_job* job = (orc_job*)arg;
  const orc_problem* pb = job->pb;
  int32_t maxL = 0;
  for (int s = 0; s < pb->S; ++s)
    if (pb->seq_lens[s] > maxL) maxL = pb->seq_lens[s];
  double* xbuf = (double*)malloc(sizeof(double) * (maxL > 0 ? maxL : 1));
  if (!xbuf) {
    pthread_mutex_lock(&job->lock);
    job->rc = ORC_ERR_NOMEM;
    pthread_mutex_unlock(&job->lock);
    return NULL;
  }
  for (;;) {
    int32_t u;
    pthread_mutex_lock(&job->lock);
    u = job->rc ? job->n_units : job->next++;
    pthread_mutex_unlock(&job->lock);
    if (u >= job->n_units) break;
    int s = job->units ? job->units[2 * u] : u / pb->Hkv;
    int h = job->units ? job->units[2 * u + 1] : u % pb->Hkv;
    int L = pb->seq_lens[s];
    for (int g = 0; g < pb->QG; ++g) {
      double* o = job->out + ((int64_t)u * pb->QG + g) * pb->D;
      double m, l;
      if (L <= 0) {
        for (int d = 0; d < pb->D; ++d) o[d] = 0.0;
        continue;
      }
      int rc = orc_attend(pb, s, h, g, 0, L, xbuf, o, &m, &l);
      if (rc) {
        pthread_mutex_lock(&job->lock);
        job->rc = rc;
        pthread_mutex_unlock(&job->lock);
        break;
      }
    }
  }
  free(xbuf);
  return NULL;
}

static int orc_check(const orc_problem* pb) {
  if (!pb->q || !pb->block_tables || !pb->seq_lens) return ORC_ERR_ARGS;
  if (pb->tq4_cache ? (!pb->centroids || (pb->D & 1))
                    : (!pb->k_cache || !pb->v_cache || !pb->kv_scales))
    return ORC_ERR_ARGS;
  if (pb->S < 1 || pb->Hkv < 1 || pb->QG < 1 || pb->D < 1 || pb->BS < 1 || pb->NB < 1 ||
      pb->max_blocks_per_seq < 1)
    return ORC_ERR_ARGS;
  if (pb->layout != ORC_LAYOUT_HEAD_MAJOR && pb->layout != ORC_LAYOUT_SLOT_MAJOR) return ORC_ERR_ARGS;
  for (int s = 0; s < pb->S; ++s) {
    int L = pb->seq_lens[s];
    if (L < 0 || (int64_t)L > (int64_t)pb->max_blocks_per_seq * pb->BS) return ORC_ERR_ARGS;
  }
  return ORC_OK;
}

/*
 * Unsplit decode attention.  `units` lists n_units (s, h) pairs (int32 pairs);
 * NULL means every (s, h) in the order s*Hkv + h.  out is [n_units][QG][D]
 * fp64, i.e. [S][Hkv*QG][D] when units is NULL.  nthreads workers share the
 * units; each unit's arithmetic is the same whatever the thread count.
 * q is bf16 bits [S][Hkv*QG][D]; softmax_scale is widened from fp32.
 */
static int orc_run(orc_problem pb, const int32_t* units, int32_t n_units, double* out,
                   int32_t nthreads);

int orc_decode(const uint16_t* q, const uint8_t* k_cache, const uint8_t* v_cache,
               const float* kv_scales, const int32_t* block_tables, const int32_t* seq_lens,
               int32_t S, int32_t Hkv, int32_t QG, int32_t D, int32_t BS, int32_t NB,
               int32_t max_blocks_per_seq, float softmax_scale, int32_t layout,
               const int32_t* units, int32_t n_units, double* out, int32_t nthreads) {
  orc_problem pb = {q, k_cache, v_cache, kv_scales, block_tables, seq_lens, S, Hkv, QG, D, BS,
                    NB, max_blocks_per_seq, (double)softmax_scale, layout, NULL, NULL};
  return orc_run(pb, units, n_units, out, nthreads);
}

/*
 * The same decode over the 4-bit record format: cache is [NB][block_bytes]
 * (block_bytes = Hkv*BS*D + Hkv*3*BS*2), centroids 16 fp32 values, q the
 * (already rotated) bf16 query.
 */
int orc_decode_tq4(const uint16_t* q, const uint8_t* cache, const float* centroids,
                   const int32_t* block_tables, const int32_t* seq_lens, int32_t S, int32_t Hkv,
                   int32_t QG, int32_t D, int32_t BS, int32_t NB, int32_t max_blocks_per_seq,
                   float softmax_scale, int32_t layout, const int32_t* units, int32_t n_units,
                   double* out, int32_t nthreads) {
  orc_problem pb = {q, NULL, NULL, NULL, block_tables, seq_lens, S, Hkv, QG, D, BS,
                    NB, max_blocks_per_seq, (double)softmax_scale, layout, cache, centroids};
  if (!cache) return ORC_ERR_ARGS;
  return orc_run(pb, units, n_units, out, nthreads);
}

/* Dequantized K and V rows (D values each) of (blk, h, slot) in the 4-bit record format. */
int orc_dequant_tq4(const uint8_t* cache, const float* centroids, int32_t Hkv, int32_t D,
                    int32_t BS, int32_t layout, int32_t blk, int32_t h, int32_t slot, double* k,
                    double* v) {
  if (!cache || !centroids || !k || !v || Hkv < 1 || D < 2 || (D & 1) || BS < 1 || blk < 0 ||
      h < 0 || h >= Hkv || slot < 0 || slot >= BS ||
      (layout != ORC_LAYOUT_HEAD_MAJOR && layout != ORC_LAYOUT_SLOT_MAJOR))
    return ORC_ERR_ARGS;
  orc_problem pb;
  memset(&pb, 0, sizeof pb);
  pb.Hkv = Hkv;
  pb.D = D;
  pb.BS = BS;
  pb.layout = layout;
  pb.tq4_cache = cache;
  pb.centroids = centroids;
  for (int d = 0; d < D; ++d) {
    k[d] = orc_tq4_kv(&pb, 0, blk, slot, h, d);
    v[d] = orc_tq4_kv(&pb, 1, blk, slot, h, d);
  }
  return ORC_OK;
}

static int orc_run(orc_problem pb, const int32_t* units, int32_t n_units, double* out,
                   int32_t nthreads) {
  int32_t S = pb.S, Hkv = pb.Hkv;
  int rc = orc_check(&pb);
  if (rc) return rc;
  if (!out) return ORC_ERR_ARGS;
  if (!units) n_units = S * Hkv;
  for (int u = 0; units && u < n_units; ++u)
    if (units[2 * u] < 0 || units[2 * u] >= S || units[2 * u + 1] < 0 || units[2 * u + 1] >= Hkv)
      return ORC_ERR_ARGS;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  orc_job job;
  job.pb = &pb;
  job.units = units;
  job.n_units = n_units;
  job.out = out;
  job.next = 0;
  job.rc = ORC_OK;
  pthread_mutex_init(&job.lock, NULL);
  if (nthreads == 1) {
    orc_worker(&job);
  } else {
    pthread_t tid[256];
    int started = 0;
    for (int i = 0; i < nthreads; ++i) {
      if (pthread_create(&tid[i], NULL, orc_worker, &job) != 0) break;
      ++started;
    }
    if (started == 0) orc_worker(&job);
    for (int i = 0; i < started; ++i) pthread_join(tid[i], NULL);
  }
  pthread_mutex_destroy(&job.lock);
  return job.rc;
}

/*
 * Split-K partials: for every (s, h, p, g) with p*E < L_s, over the tokens
 * [p*E, min((p+1)*E, L_s)):  o[s][h][p][g][D] = normalised partial output,
 * m[s][h][p][g] = max scaled logit, l[s][h][p][g] = sum exp(x - m).
 * Entries of dead partitions (p*E >= L_s) are left untouched.
 */
int orc_partials(const uint16_t* q, const uint8_t* k_cache, const uint8_t* v_cache,
                 const float* kv_scales, const int32_t* block_tables, const int32_t* seq_lens,
                 int32_t S, int32_t Hkv, int32_t QG, int32_t D, int32_t BS, int32_t NB,
                 int32_t max_blocks_per_seq, float softmax_scale, int32_t layout, int32_t P,
                 int32_t E, double* o, double* m, double* l) {
  orc_problem pb = {q, k_cache, v_cache, kv_scales, block_tables, seq_lens, S, Hkv, QG, D, BS,
                    NB, max_blocks_per_seq, (double)softmax_scale, layout, NULL, NULL};
  int rc = orc_check(&pb);
  if (rc) return rc;
  if (P < 1 || E < 1 || !o || !m || !l) return ORC_ERR_ARGS;
  int32_t maxL = 0;
  for (int s = 0; s < S; ++s)
    if (seq_lens[s] > maxL) maxL = seq_lens[s];
  if ((int64_t)maxL > (int64_t)P * E) return ORC_ERR_ARGS;
  double* xbuf = (double*)malloc(sizeof(double) * (E > 0 ? E : 1));
  if (!xbuf) return ORC_ERR_NOMEM;
  for (int s = 0; s < S && !rc; ++s) {
    int L = seq_lens[s];
    for (int h = 0; h < Hkv && !rc; ++h)
      for (int p = 0; p < P && !rc; ++p) {
        int t0 = p * E, t1 = (p + 1) * E < L ? (p + 1) * E : L;
        if (t0 >= L) continue;
        for (int g = 0; g < QG && !rc; ++g) {
          int64_t r = (((int64_t)s * Hkv + h) * P + p) * QG + g;
          rc = orc_attend(&pb, s, h, g, t0, t1, xbuf, o + r * D, &m[r], &l[r]);
        }
      }
  }
  free(xbuf);
  return rc;
}

/*
 * Log-sum-exp merge of split-K partials (layout of orc_partials) into
 * out[S][Hkv*QG][D]: over live partitions p (p*E < L_s),
 * M = max m_p, w_p = l_p exp(m_p - M), out = sum w_p o_p / sum w_p.
 * L_s = 0 gives zeros.
 */
int orc_merge(const double* o, const double* m, const double* l, const int32_t* seq_lens,
              int32_t S, int32_t Hkv, int32_t QG, int32_t D, int32_t P, int32_t E, double* out) {
  if (!o || !m || !l || !seq_lens || !out || S < 1 || Hkv < 1 || QG < 1 || D < 1 || P < 1 || E < 1)
    return ORC_ERR_ARGS;
  for (int s = 0; s < S; ++s) {
    int L = seq_lens[s];
    int live = L <= 0 ? 0 : (L + E - 1) / E;
    if (live > P) return ORC_ERR_ARGS;
    for (int h = 0; h < Hkv; ++h)
      for (int g = 0; g < QG; ++g) {
        double* dst = out + (((int64_t)s * Hkv + h) * QG + g) * D;
        double M = -INFINITY, W = 0.0;
        for (int d = 0; d < D; ++d) dst[d] = 0.0;
        if (live == 0) continue;
        for (int p = 0; p < live; ++p) {
          double mp = m[(((int64_t)s * Hkv + h) * P + p) * QG + g];
          if (mp > M) M = mp;
        }
        for (int p = 0; p < live; ++p) {
          int64_t r = (((int64_t)s * Hkv + h) * P + p) * QG + g;
          double w = l[r] * exp(m[r] - M);
          W += w;
          for (int d = 0; d < D; ++d) dst[d] += w * o[r * D + d];
        }
        for (int d = 0; d < D; ++d) dst[d] /= W;
      }
  }
  return ORC_OK;
}

/*
 * KV-cache writer (the step upstream of decode that fills the cache this
 * oracle reads; the per-block scale region follows the fp8 record writer of
 * page "vllm.models.deepseek_v41.amd.mono.attention.front", stage_qkv, with
 * this library's scale rule).  For each new token t with slot_mapping[t] >= 0
 * (slot = block * BS + offset) and each kv head h, the K row and the V row
 * (bf16, 128 values each) are quantized on their own:
 *   s = absmax / 448        (fp32 division: the quantizer's integer decisions
 *   q_d = x_d / s            are taken in fp32, as the GPU writer takes them)
 *   code_d = e4m3fn(q_d), round to nearest, ties to even, saturating at 448;
 *   absmax = 0 gives s = 0 and codes 0.
 * Codes go to k_cache / v_cache[block][h][offset][:], s to
 * kv_scales[block][h][field][offset]; nothing else is touched.
 */

/* Nearest e4m3fn code of a finite fp32 value, ties to the code with an even
 * mantissa: a plain search over the 127 non-negative finite codes, using the
 * closed-form decoder above.  The search only sees finite codes, so a
 * magnitude above 448 saturates to +-448 by construction. */
uint8_t orc_enc_e4m3fn(float x) {
  double ax = fabs((double)x);
  int best = 0;
  double best_err = INFINITY;
  for (int c = 0; c <= 0x7E; ++c) {
    double err = fabs(orc_dec_e4m3fn((uint8_t)c) - ax);
    if (err < best_err || (err == best_err && (c & 1) == 0)) {
      best = c;
      best_err = err;
    }
  }
  return (uint8_t)((signbit(x) ? 0x80 : 0x00) | best);
}

int orc_kv_write(const uint16_t* k_new, const uint16_t* v_new, const int32_t* slot_mapping,
                 int32_t T, int32_t Hkv, int32_t D, int32_t BS, int32_t NB, int32_t layout,
                 uint8_t* k_cache, uint8_t* v_cache, float* kv_scales) {
  if (!k_new || !v_new || !slot_mapping || !k_cache || !v_cache || !kv_scales || T < 0 ||
      Hkv < 1 || D < 1 || BS < 1 || NB < 1 ||
      (layout != ORC_LAYOUT_HEAD_MAJOR && layout != ORC_LAYOUT_SLOT_MAJOR))
    return ORC_ERR_ARGS;
  for (int t = 0; t < T; ++t) {
    int32_t slot = slot_mapping[t];
    if (slot < 0) continue;
    if ((int64_t)slot >= (int64_t)NB * BS) return ORC_ERR_BLOCK;
    int blk = slot / BS, off = slot % BS;
    for (int h = 0; h < Hkv; ++h)
      for (int field = 0; field < 2; ++field) {
        const uint16_t* src = (field == 0 ? k_new : v_new) + ((int64_t)t * Hkv + h) * D;
        uint8_t* dst = (field == 0 ? k_cache : v_cache) + orc_row(layout, Hkv, BS, blk, h, off) * D;
        float absmax = 0.0f;
        for (int d = 0; d < D; ++d) {
          float x = (float)orc_dec_bf16(src[d]);
          if (fabsf(x) > absmax) absmax = fabsf(x);
        }
        float s = absmax / 448.0f;
        for (int d = 0; d < D; ++d) {
          float x = (float)orc_dec_bf16(src[d]);
          dst[d] = s > 0.0f ? orc_enc_e4m3fn(x / s) : 0;
        }
        kv_scales[(((int64_t)blk * Hkv + h) * 2 + field) * BS + off] = s;
      }
  }
  return ORC_OK;
}
