/*
 * nvfp4_ref.c - plain C form of the CPU oracle's NVFP4 quantizer and decoder.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the cpu_baseline leg of
 * bench.py may load this library (through oracle/nvfp4_ref.py).  It shares nothing with the HIP
 * library: no header, no table, no helper.  It exists because the NumPy oracle needs ~80 ns per
 * element, which is too slow for the full-size workloads (up to 17 G weight elements); this is the
 * same definition, written out element by element.
 *
 * What it computes (nvfp4-megamoe-kernel CURRENT_BUG.md@2fc81cc, "Root Cause" and "Key evidence":
 * the FP4 quantizer multiplies the tensor by a global scale before forming the FP8 block scales,
 * and a scale that ignores the tensor's amax overflows them; CURRENT_BUG.md@2e65594, "Test Plan"
 * Phase 1: activations are quantized to NVFP4 before each grouped GEMM):
 *   amax   = max |x| over the valid rows
 *   gs     = fl32(2688 / amax), 2688 = 448 (largest E4M3) * 6 (largest E2M1); 1 when amax = 0
 *   per block of 16 consecutive elements of a row:
 *     scale = OCP E4M3FN nearest to block_amax * gs / 6, ties to the even code, saturating at 448
 *     code  = sign of x | index of the E2M1 magnitude {0,.5,1,1.5,2,3,4,6} nearest to
 *             |x| * gs / scale, ties to the even index; magnitude 0 when the scale is 0
 *   two codes per byte, the even element in the low nibble; invalid rows get zero bytes.
 * Exactness: every product compared here is exact in double (a bf16 value times an fp32 scale has
 * at most 32 significant bits; a grid midpoint times an E4M3 value at most 7), so each rounding
 * decision is taken on exact values and no division is rounded.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* E2M1 magnitudes by the code's low 3 bits. */
static const double kE2M1[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

/* OCP E4M3FN value of a code without its sign bit (0x00..0x7E): 4 exponent bits with bias 7 and
 * 3 mantissa bits; exponent 0 is the subnormal range m * 2^-9. */
static double e4m3_value(int c) {
  const int e = (c >> 3) & 0xF, m = c & 7;
  return e == 0 ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
}

static double bf16_value(uint16_t b) {
  const uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* 6 * value of every finite non-negative E4M3 code, in code order (increasing), built once. */
static double g_six_grid[127];
static pthread_once_t g_grid_once = PTHREAD_ONCE_INIT;
static void build_grid(void) {
  for (int c = 0; c < 127; ++c) g_six_grid[c] = 6.0 * e4m3_value(c);
}

/* E4M3 code nearest to p / 6 (p exact), ties to the even code, saturating at 448 (0x7E).  Works on
 * p against 6 * grid values and 6 * midpoints = 3 * (lower + upper), all exact. */
static int block_scale_code(double p) {
  if (p >= g_six_grid[0x7E]) return 0x7E;
  int lo = 0, hi = 0x7E; /* 6 * grid[lo] <= p < 6 * grid[hi] */
  while (hi - lo > 1) {
    const int mid = (lo + hi) / 2;
    if (g_six_grid[mid] <= p) lo = mid;
    else hi = mid;
  }
  const double six_mid = 0.5 * (g_six_grid[lo] + g_six_grid[hi]);
  if (p < six_mid) return lo;
  if (p > six_mid) return hi;
  return (lo % 2 == 0) ? lo : hi;
}

/* Midpoints between consecutive E2M1 magnitudes times the block scale value s (exact). */
static void thresholds(double s, double t[7]) {
  for (int j = 0; j < 7; ++j) t[j] = 0.5 * (kE2M1[j] + kE2M1[j + 1]) * s;
}

/* 4-bit code of x with global scale gs, for a block whose scale value s gave thresholds t. */
static int element_code(double x, double gs, double s, const double t[7]) {
  int mag = 0;
  if (s != 0.0) {
    const double a = fabs(x) * gs;
    for (int j = 0; j < 7; ++j)
      /* past the midpoint between magnitudes j and j+1; at a tie the even index wins (up when
       * j + 1 is even) */
      if (a > t[j] || (a == t[j] && ((j + 1) % 2 == 0))) mag = j + 1;
  }
  return (signbit(x) ? 8 : 0) | mag;
}

float nvfp4_ref_global_scale(double amax) {
  if (amax == 0.0) return 1.0f;
  return 2688.0f / (float)amax; /* IEEE single division: the exact quotient rounded once */
}

/* ---- row-parallel drivers ---------------------------------------------------------------------- */
typedef struct {
  const uint16_t* x;
  const uint8_t* codes_in;
  const uint8_t* scales_in;
  const uint8_t* valid;
  int64_t cols, r0, r1;
  double gs;
  uint8_t* codes;
  uint8_t* scales;
  double* out;
  double amax;
} Job;

static void* amax_job(void* arg) {
  Job* j = (Job*)arg;
  double m = 0.0;
  for (int64_t r = j->r0; r < j->r1; ++r) {
    if (j->valid && !j->valid[r]) continue;
    for (int64_t c = 0; c < j->cols; ++c) {
      const double v = fabs(bf16_value(j->x[r * j->cols + c]));
      if (v > m) m = v;
    }
  }
  j->amax = m;
  return NULL;
}

static void* quant_job(void* arg) {
  Job* j = (Job*)arg;
  const int64_t nb = j->cols / 16;
  for (int64_t r = j->r0; r < j->r1; ++r) {
    uint8_t* crow = j->codes + r * (j->cols / 2);
    uint8_t* srow = j->scales + r * nb;
    if (j->valid && !j->valid[r]) {
      memset(crow, 0, (size_t)(j->cols / 2));
      memset(srow, 0, (size_t)nb);
      continue;
    }
    for (int64_t b = 0; b < nb; ++b) {
      const uint16_t* xb = j->x + r * j->cols + 16 * b;
      double bmax = 0.0;
      for (int i = 0; i < 16; ++i) {
        const double v = fabs(bf16_value(xb[i]));
        if (v > bmax) bmax = v;
      }
      const int sc = block_scale_code(bmax * j->gs);
      const double s = e4m3_value(sc);
      double t[7];
      thresholds(s, t);
      srow[b] = (uint8_t)sc;
      for (int i = 0; i < 16; i += 2) {
        const int c0 = element_code(bf16_value(xb[i]), j->gs, s, t);
        const int c1 = element_code(bf16_value(xb[i + 1]), j->gs, s, t);
        crow[8 * b + i / 2] = (uint8_t)(c0 | (c1 << 4));
      }
    }
  }
  return NULL;
}

static void* dequant_job(void* arg) {
  Job* j = (Job*)arg;
  const int64_t nb = j->cols / 16;
  for (int64_t r = j->r0; r < j->r1; ++r) {
    for (int64_t b = 0; b < nb; ++b) {
      const int sc = j->scales_in[r * nb + b];
      const double s = (sc & 0x7F) == 0x7F ? NAN : ((sc & 0x80) ? -1.0 : 1.0) * e4m3_value(sc & 0x7F);
      for (int i = 0; i < 16; ++i) {
        const int64_t k = 16 * b + i;
        const uint8_t byte = j->codes_in[r * (j->cols / 2) + k / 2];
        const int code = (k % 2 == 0) ? (byte & 0xF) : (byte >> 4);
        const double v = ((code & 8) ? -1.0 : 1.0) * kE2M1[code & 7];
        j->out[r * j->cols + k] = v * s;
      }
    }
  }
  return NULL;
}

static void run_rows(Job* proto, int64_t rows, int nthreads, void* (*fn)(void*), double* amax_out) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if ((int64_t)nthreads > rows) nthreads = rows > 0 ? (int)rows : 1;
  Job jobs[256];
  pthread_t th[256];
  for (int t = 0; t < nthreads; ++t) {
    jobs[t] = *proto;
    jobs[t].r0 = rows * t / nthreads;
    jobs[t].r1 = rows * (t + 1) / nthreads;
    jobs[t].amax = 0.0;
  }
  int created[256] = {0};
  for (int t = 1; t < nthreads; ++t) {
    created[t] = pthread_create(&th[t], NULL, fn, &jobs[t]) == 0;
    if (!created[t]) fn(&jobs[t]); /* no thread: do that share here */
  }
  fn(&jobs[0]);
  for (int t = 1; t < nthreads; ++t)
    if (created[t]) pthread_join(th[t], NULL);
  if (amax_out) {
    double m = 0.0;
    for (int t = 0; t < nthreads; ++t)
      if (jobs[t].amax > m) m = jobs[t].amax;
    *amax_out = m;
  }
}

/* amax over the valid rows (valid may be NULL: all rows) of bf16 x [rows, cols]. */
double nvfp4_ref_amax(const uint16_t* x, int64_t rows, int64_t cols, const uint8_t* valid, int nthreads) {
  Job p;
  memset(&p, 0, sizeof p);
  p.x = x;
  p.cols = cols;
  p.valid = valid;
  double m = 0.0;
  if (rows > 0 && cols > 0) run_rows(&p, rows, nthreads, amax_job, &m);
  return m;
}

/* Quantize bf16 x [rows, cols] (cols a multiple of 16) with global scale gs: codes [rows, cols/2],
 * scales [rows, cols/16]; rows with valid[r] == 0 get zero bytes.  Returns 0, or -1 on bad sizes. */
int nvfp4_ref_quantize(const uint16_t* x, int64_t rows, int64_t cols, const uint8_t* valid, float gs,
                       uint8_t* codes, uint8_t* scales, int nthreads) {
  if (rows < 0 || cols <= 0 || cols % 16 != 0) return -1;
  pthread_once(&g_grid_once, build_grid);
  Job p;
  memset(&p, 0, sizeof p);
  p.x = x;
  p.cols = cols;
  p.valid = valid;
  p.gs = (double)gs;
  p.codes = codes;
  p.scales = scales;
  if (rows > 0) run_rows(&p, rows, nthreads, quant_job, NULL);
  return 0;
}

/* Exact value of every element before the global scale: e2m1(code) * e4m3(scale) (NaN for the
 * E4M3 NaN codes).  out [rows, cols] float64.  Returns 0, or -1 on bad sizes. */
int nvfp4_ref_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols, double* out,
                         int nthreads) {
  if (rows < 0 || cols <= 0 || cols % 16 != 0) return -1;
  Job p;
  memset(&p, 0, sizeof p);
  p.codes_in = codes;
  p.scales_in = scales;
  p.cols = cols;
  p.out = out;
  if (rows > 0) run_rows(&p, rows, nthreads, dequant_job, NULL);
  return 0;
}
