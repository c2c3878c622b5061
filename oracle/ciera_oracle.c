/*
 * ciera_oracle.c -- CPU oracle for the lossless BF16 codec.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, scalar reference
 * that the HIP library is checked against.  Only the tests, the smoke check
 * and the benchmark's CPU-baseline leg load it.  The HIP library never
 * includes, links or calls anything here, and nothing here comes from the
 * HIP sources: the two sides share no code, header, table or constant.
 *
 * What it computes (every step in element order, one value at a time):
 *
 *  - Field split.  A BF16 value is 1 sign bit, 8 exponent bits and 7 mantissa
 *    bits.  Sign and mantissa stay together as one raw byte (sign in bit 7);
 *    the exponent is handled on its own.  ZipCCL research digest, section 3.1
 *    (first paragraph); CIERA page, section 3.1 (the sender splits every value
 *    into exponent bits and sign-plus-mantissa bits).
 *
 *  - Window.  sigma comes from the tensor's standard deviation (sample
 *    variance, correction 1, over the finite values).  The 7-binade window
 *    starts at the integer nearest x_opt = log2(sigma) + 0.5*log2(14 ln2 /
 *    16383).  ZipCCL digest, section 3.1, the P_win equation, the x_opt
 *    equation and Figure 2.  Written as a comparison of the variance with the
 *    thresholds K0 * 4^k, K0 = 16383 / (28 ln 2), so no logarithm is taken:
 *    k = floor(x_opt + 1/2)  <=>  var >= K0 * 4^k.
 *
 *  - 3-bit code.  An exponent E in [E0, E0+6] gets code E-E0+1 (1..7); any
 *    other exponent gets code 0 and its full 8 bits go to the escape list, in
 *    element order.  ZipCCL digest, section 3.1 (codes 001..111, code 000 plus
 *    the full exponent in a separate zero-point list).
 *
 *  - Exponent reuse (ciera mode only).  The shard is cut into blocks of B
 *    values counted from the shard start.  A block is "changed" when any of
 *    its exponents differs from the sender's exponent cache (the exponents
 *    sent for the previous iteration).  Only changed blocks send exponents; a
 *    one-bit-per-block bitmap marks them; sign+mantissa of every value is sent.
 *    The receiver takes unchanged blocks' exponents from its own cache.  CIERA
 *    page, section 3.1 (bitmap, sender and receiver caches) and section 3.2
 *    (payload S_{s+m} + S_bm + q S_e).  The cache here holds the exponents
 *    themselves, compared exactly, in place of the page's per-block hash.
 *
 *  - Block hash (the page's sender state, section 3.1: a 128-bit hash per
 *    block made of two independent 64-bit SplitMix64 hashes; a block counts
 *    as unchanged only when its hash equals the stored one).  The page does
 *    not say how a block's bytes enter SplitMix64.  Here: the block's
 *    exponent fields, 8 at a time, form little-endian 64-bit words w_k (the
 *    last word of a short block filled with zeros); hash h is the sum mod
 *    2^64, over the words that are not zero, of mix(w_k + s_h + (k+1) g_h),
 *    where mix is SplitMix64's output function, i.e. the (k+1)-th output of
 *    a SplitMix64 generator with seed w_k + s_h and increment g_h.  Hash 0
 *    uses seed 0 and SplitMix64's own increment; hash 1 its own seed and odd
 *    increment.  An all-zero block hashes to (0, 0), so an all-zero hash
 *    cache stands for all-zero previous exponents, as an all-zero exponent
 *    cache does.
 *
 *  - Packing.  The stream is cut into chunks of 65,536 input values; each
 *    chunk is written as a self-contained segment whose sections start on
 *    128-byte boundaries, and the three code bits go to three 1-bit arrays.
 *    ZipCCL digest, section 3.1 (last paragraph: chunks padded to 128 bytes,
 *    codes as three aligned 1-bit arrays) and Figure 1 (codec writes the
 *    collective's chunk layout; only a size exchange is added).
 *
 * Parity unpinned by the pages: the byte layout below (the pages print no
 * encoded bytes; the tests pin it only by the closed-form stream size and a
 * second, independent encoder), the rANS variant's format and parameters
 * further down (the CIERA page names an ANS coder and gives no parameters;
 * pinned by a second encoder, a worked normalisation and the information
 * content), and hash 1's seed and increment (chosen here: the pages give
 * none; both hashes are pinned by value against an independent
 * implementation of the construction below, hash 0 also against
 * SplitMix64's published outputs).  Every value the pages do fix (fields,
 * window, codes, reuse, SplitMix64) is pinned by the tests against the
 * pages, and the largest-stream bound against the closed-form size at full
 * counts and a stream that attains it.
 *
 * Byte layout (all integers little-endian, all unnamed bytes zero):
 *
 *   header, 128 bytes:
 *     0  char[4] magic "ZIP3" (zip3 mode) or "CIER" (ciera mode)
 *     4  u16 version = 1
 *     6  u8  mode (0 zip3, 1 ciera)
 *     7  u8  E0 (window base; codes 1..7 mean E0..E0+6)
 *     8  u64 n (values)
 *     16 u32 B (0 in zip3 mode)
 *     20 u32 C = 65536 (values per chunk)
 *     24 u64 nchunks = ceil(n / C)
 *     32 u64 total_bytes
 *     40 u64 n_changed_blocks (ciera; in zip3 mode 0)
 *     48 u64 n_escapes
 *   chunk table at byte 128: nchunks+1 u64 absolute offsets (the last one is
 *     total_bytes);
 *   escape index right after it: for each chunk, four u16 giving the number of
 *     escapes among the chunk's values before value 0, 16384, 32768 and
 *     49152 of the chunk (a seek index: a decoder can start at any quarter of
 *     a chunk); table and index together zero-padded to a 128-byte multiple.
 *   chunk c (values [cC, min(cC+C, n)), n_c of them), each section padded to
 *   a multiple of 128 bytes with zeros:
 *     1. sm:     n_c bytes, sm = (sign << 7) | mantissa
 *     2. bitmap: ciera only, ceil(nb_c / 8) bytes, nb_c = ceil(n_c / B);
 *                bit (j & 7) of byte (j >> 3) set when block j of the chunk
 *                is changed
 *     3. planes: three arrays of P_c bytes; plane b holds bit b of the code
 *                of slot t in bit (t & 7) of byte (t >> 3).  zip3: slot t is
 *                value t of the chunk, P_c = ceil(n_c / 8).  ciera: the r-th
 *                changed block of the chunk owns slots rB .. rB+B-1, slot
 *                rB+s is value s of that block (0 past the end of the data),
 *                P_c = (changed blocks of the chunk) * B / 8.
 *     4. escapes: one byte (the raw exponent) per code-0 slot that holds a
 *                value, in slot order.
 *
 * The statistic is exact.  Every finite BF16 value is an integer significand
 * M (|M| <= 255, the hidden bit included) times 2^(E'-134), E' = max(E, 1).
 * Per exponent field E the oracle sums M and M^2 in 64-bit integers, so the
 * sums do not depend on the order of the values; the variance
 * (n S2 - S1^2) / (n (n - 1)) is then formed and compared with the
 * thresholds K0 * 4^k in fixed-size integer arithmetic (768-bit, enough for
 * n <= 2^40), with K0 taken as the double nearest 16383 / (28 ln 2).
 * No rounding happens anywhere, so a chunk-parallel run that adds the same
 * integer sums gives the same window.
 *
 * orc_encode_mt / orc_decode_mt run the same per-chunk steps as orc_encode /
 * orc_decode on several threads (chunks are self-contained segments; their
 * offsets come from the closed-form size of each chunk, checked against what
 * the chunk's writer returns).  They exist to time the oracle on all host
 * cores and to check full-size tensors quickly; their output is byte-equal
 * to the single-threaded functions', which the tests check.
 */
#include <math.h>
#include <pthread.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum {
  ORC_OK = 0,
  ORC_ERR_ARG = 1,
  ORC_ERR_CAPACITY = 2,
  ORC_ERR_FORMAT = 5,
  ORC_ERR_NOMEM = 6
};

#define ORC_CHUNK 65536ull
#define ORC_QUARTER 16384ull /* escape index granularity */
#define ORC_HEADER 128ull
#define ORC_MAX_N (1ull << 40)

/* 16383 / (28 ln 2), rounded to the nearest double. */
static const double ORC_K0 = 0x1.a610ca4a234eep+9;

static uint64_t pad128(uint64_t x) { return (x + 127ull) / 128ull * 128ull; }
static uint64_t ceil_div(uint64_t a, uint64_t b) { return (a + b - 1) / b; }

/* Byte offset of the escape index and of the first chunk. */
static uint64_t index_pos(uint64_t nchunks) { return ORC_HEADER + 8ull * (nchunks + 1ull); }
static uint64_t payload_pos(uint64_t nchunks) { return ORC_HEADER + pad128(8ull * (nchunks + 1ull) + 8ull * nchunks); }

static unsigned exp_field(uint16_t v) { return (v >> 7) & 0xFFu; }
static unsigned sm_field(uint16_t v) { return ((unsigned)(v >> 15) << 7) | (v & 0x7Fu); }
static uint16_t join_fields(unsigned sm, unsigned e) {
  return (uint16_t)(((sm >> 7) << 15) | (e << 7) | (sm & 0x7Fu));
}

static void put_u16(uint8_t* p, unsigned v) {
  p[0] = (uint8_t)v;
  p[1] = (uint8_t)(v >> 8);
}
static void put_u32(uint8_t* p, uint32_t v) {
  for (int i = 0; i < 4; i++) p[i] = (uint8_t)(v >> (8 * i));
}
static void put_u64(uint8_t* p, uint64_t v) {
  for (int i = 0; i < 8; i++) p[i] = (uint8_t)(v >> (8 * i));
}
static unsigned get_u16(const uint8_t* p) { return (unsigned)p[0] | ((unsigned)p[1] << 8); }
static uint32_t get_u32(const uint8_t* p) {
  uint32_t v = 0;
  for (int i = 3; i >= 0; i--) v = (v << 8) | p[i];
  return v;
}
static uint64_t get_u64(const uint8_t* p) {
  uint64_t v = 0;
  for (int i = 7; i >= 0; i--) v = (v << 8) | p[i];
  return v;
}

/* Exact value of a finite BF16 bit pattern.  Normal: (128+m) * 2^(E-134);
 * subnormal (E = 0): m * 2^-133.  Both are exact in double. */
double orc_bf16_value(uint16_t v) {
  unsigned e = exp_field(v);
  unsigned m = v & 0x7Fu;
  double mag = (e == 0) ? ldexp((double)m, -133) : ldexp((double)(128u + m), (int)e - 134);
  return (v & 0x8000u) ? -mag : mag;
}

/* ---- exact window statistic ---------------------------------------------
 * ZipCCL digest, section 3.1: sigma comes from one standard-deviation call
 * over the tensor (sample variance, correction 1); NaN and +-Inf (exponent
 * field 255) are left out, since a plain std of them is NaN.
 *
 * A finite value is M 2^(E'-134) with M = +-(128 + m) for E >= 1, M = +-m
 * for E = 0, and E' = max(E, 1).  a[E] = sum of M and b[E] = sum of M^2 over
 * the finite values with exponent field E (|a| < 2^48, b < 2^56 for
 * n <= 2^40).  Scaled by 2^133 and 2^266, the sums of the values and of their
 * squares are the integers s1 = sum a[E] 2^(E'-1) (< 2^310 in magnitude)
 * and s2 = sum b[E] 2^(2E'-2) (< 2^570), and
 *     var = (nf s2 - s1^2) / (nf (nf - 1) 2^266).
 * With K0 = K0m 2^-43 (K0m the 53-bit integer significand of the double),
 *     var >= K0 4^k  <=>  nf s2 - s1^2 >= K0m nf (nf - 1) 2^(223 + 2k),
 * both sides below 2^660 for every k in [-127, 122]. */
#define BN_LIMBS 24 /* 768 bits */
typedef struct {
  uint32_t w[BN_LIMBS]; /* little-endian 32-bit limbs */
} bn_t;

static void bn_from_u64(bn_t* a, uint64_t v) {
  memset(a, 0, sizeof(*a));
  a->w[0] = (uint32_t)v;
  a->w[1] = (uint32_t)(v >> 32);
}

static void bn_shl(bn_t* a, unsigned sh) {
  const unsigned limbs = sh / 32u, bits = sh % 32u;
  for (int i = BN_LIMBS - 1; i >= 0; i--) {
    uint64_t hi = (i - (int)limbs >= 0) ? a->w[i - limbs] : 0u;
    uint64_t lo = (i - (int)limbs - 1 >= 0) ? a->w[i - limbs - 1] : 0u;
    a->w[i] = (uint32_t)(((hi << 32 | lo) << bits) >> 32);
  }
}

static void bn_add(bn_t* a, const bn_t* b) {
  uint64_t carry = 0;
  for (int i = 0; i < BN_LIMBS; i++) {
    carry += (uint64_t)a->w[i] + b->w[i];
    a->w[i] = (uint32_t)carry;
    carry >>= 32;
  }
}

/* a -= b; requires a >= b. */
static void bn_sub(bn_t* a, const bn_t* b) {
  int64_t borrow = 0;
  for (int i = 0; i < BN_LIMBS; i++) {
    int64_t d = (int64_t)a->w[i] - (int64_t)b->w[i] - borrow;
    borrow = d < 0;
    a->w[i] = (uint32_t)(d + (borrow << 32));
  }
}

static int bn_cmp(const bn_t* a, const bn_t* b) {
  for (int i = BN_LIMBS - 1; i >= 0; i--)
    if (a->w[i] != b->w[i]) return a->w[i] < b->w[i] ? -1 : 1;
  return 0;
}

/* r = a * b; the operands' sizes keep the product below 2^768. */
static void bn_mul(bn_t* r, const bn_t* a, const bn_t* b) {
  uint32_t acc[2 * BN_LIMBS];
  memset(acc, 0, sizeof(acc));
  for (int i = 0; i < BN_LIMBS; i++) {
    uint64_t carry = 0;
    for (int j = 0; j < BN_LIMBS; j++) {
      carry += (uint64_t)a->w[i] * b->w[j] + acc[i + j];
      acc[i + j] = (uint32_t)carry;
      carry >>= 32;
    }
    acc[i + BN_LIMBS] = (uint32_t)carry;
  }
  memcpy(r->w, acc, sizeof(r->w));
}

static void bn_mul_u64(bn_t* a, uint64_t m) {
  bn_t t;
  bn_from_u64(&t, m);
  bn_t r;
  bn_mul(&r, a, &t);
  *a = r;
}

/* Per exponent field: the sum of the signed significands and of their
 * squares over the finite values, and the number of finite values.  a and b
 * have 256 entries (entry 255 stays 0). */
void orc_exponent_sums(const uint16_t* x, uint64_t n, int64_t* a, uint64_t* b, uint64_t* nfinite) {
  memset(a, 0, 256 * sizeof(int64_t));
  memset(b, 0, 256 * sizeof(uint64_t));
  uint64_t nf = 0;
  for (uint64_t i = 0; i < n; i++) {
    const unsigned e = exp_field(x[i]);
    if (e == 255u) continue;
    const int64_t mag = (int64_t)((e == 0u ? 0u : 128u) + (x[i] & 0x7Fu));
    a[e] += (x[i] & 0x8000u) ? -mag : mag;
    b[e] += (uint64_t)(mag * mag);
    nf++;
  }
  *nfinite = nf;
}

/* Window base from exact sums (see above): E0 = clamp(127 + k, 0, 249) for
 * the largest k with var >= K0 4^k; E0 = 0 when nf < 2 or var = 0. */
int orc_window_base_exact(const int64_t* a, const uint64_t* b, uint64_t nf) {
  if (nf < 2) return 0;
  bn_t pos, neg, s2, t;
  bn_from_u64(&pos, 0);
  bn_from_u64(&neg, 0);
  bn_from_u64(&s2, 0);
  for (unsigned e = 0; e < 255u; e++) {
    const unsigned ep = e ? e : 1u;
    if (a[e] != 0) {
      bn_from_u64(&t, a[e] > 0 ? (uint64_t)a[e] : (uint64_t)(-a[e]));
      bn_shl(&t, ep - 1u);
      bn_add(a[e] > 0 ? &pos : &neg, &t);
    }
    bn_from_u64(&t, b[e]);
    bn_shl(&t, 2u * ep - 2u);
    bn_add(&s2, &t);
  }
  /* |s1| = |pos - neg| */
  bn_t s1 = pos;
  if (bn_cmp(&pos, &neg) >= 0) {
    bn_sub(&s1, &neg);
  } else {
    s1 = neg;
    bn_sub(&s1, &pos);
  }
  bn_t d, sq;
  d = s2;
  bn_mul_u64(&d, nf);
  bn_mul(&sq, &s1, &s1);
  bn_sub(&d, &sq); /* nf s2 - s1^2 >= 0 (Cauchy-Schwarz) */
  bn_t zero;
  bn_from_u64(&zero, 0);
  if (bn_cmp(&d, &zero) == 0) return 0;

  int exp2;
  const double mant = frexp(ORC_K0, &exp2);          /* K0 = mant 2^exp2, mant in [1/2, 1) */
  const uint64_t k0m = (uint64_t)ldexp(mant, 53);   /* exact: a 53-bit integer */
  const int k0e = exp2 - 53;                         /* K0 = k0m 2^k0e (k0e = -43) */
  int e0 = 0;
  for (int k = -127; k <= 122; k++) {
    /* var >= K0 4^k  <=>  d 2^266 ... rearranged: d >= k0m nf (nf-1) 2^(266 + k0e + 2k) */
    const int sh = 266 + k0e + 2 * k;
    bn_t lhs = d, rhs;
    bn_from_u64(&rhs, k0m);
    bn_mul_u64(&rhs, nf);
    bn_mul_u64(&rhs, nf - 1u);
    if (sh >= 0)
      bn_shl(&rhs, (unsigned)sh);
    else
      bn_shl(&lhs, (unsigned)(-sh));
    if (bn_cmp(&lhs, &rhs) >= 0) e0 = 127 + k;
  }
  return e0;
}

/* Window base for a given variance (a double, so K0 4^k and the comparison
 * are exact): the largest k with var >= K0 4^k, E0 = clamp(127 + k, 0, 249);
 * E0 = 0 for fewer than two finite values or var <= 0. */
int orc_window_base(double var, uint64_t nfinite) {
  if (nfinite < 2 || !(var > 0.0)) return 0;
  int e0 = 0;
  for (int k = -127; k <= 122; k++) {
    if (var >= ldexp(ORC_K0, 2 * k)) e0 = 127 + k;
  }
  return e0;
}

int orc_choose_e0(const uint16_t* x, uint64_t n) {
  int64_t a[256];
  uint64_t b[256], nf;
  orc_exponent_sums(x, n, a, b, &nf);
  return orc_window_base_exact(a, b, nf);
}

/* SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
 * generators", OOPSLA 2014): the state advances by an odd increment and each
 * output is the new state through a fixed mixing function (two xor-shift
 * multiply rounds and a final xor-shift). */
#define ORC_SM64_GAMMA 0x9E3779B97F4A7C15ull

static uint64_t sm64_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

uint64_t orc_splitmix64_next(uint64_t* state) {
  *state += ORC_SM64_GAMMA;
  return sm64_mix(*state);
}

/* The block hashes (two u64 per block, block b at out[2b], out[2b+1]) of
 * x's exponent fields: see "Block hash" at the top of this file. */
static const uint64_t ORC_HASH_SEED[2] = {0ull, 0x243F6A8885A308D3ull};
static const uint64_t ORC_HASH_GAMMA[2] = {ORC_SM64_GAMMA, 0xD1B54A32D192ED03ull};

void orc_block_hashes(const uint16_t* x, uint64_t n, uint32_t B, uint64_t* out) {
  uint64_t nb = ceil_div(n, B);
  for (uint64_t b = 0; b < nb; b++) {
    uint64_t begin = b * B;
    uint64_t end = (begin + B < n) ? begin + B : n;
    uint64_t h[2] = {0ull, 0ull};
    for (uint64_t k = 0; begin + 8ull * k < end; k++) {
      uint64_t w = 0;
      for (unsigned i = 0; i < 8u && begin + 8ull * k + i < end; i++)
        w |= (uint64_t)exp_field(x[begin + 8ull * k + i]) << (8u * i);
      if (w == 0) continue;
      for (int j = 0; j < 2; j++) h[j] += sm64_mix(w + ORC_HASH_SEED[j] + (k + 1ull) * ORC_HASH_GAMMA[j]);
    }
    out[2 * b] = h[0];
    out[2 * b + 1] = h[1];
  }
}

static unsigned code_of(unsigned e, unsigned e0) {
  return (e >= e0 && e <= e0 + 6u) ? e - e0 + 1u : 0u;
}

static int valid_block_size(uint32_t B) {
  return B >= 64u && B <= (uint32_t)ORC_CHUNK && (B & (B - 1u)) == 0u;
}

/* Largest stream encode can produce for n values (every block changed, every
 * value an escape).  B = 0 selects zip3 mode. */
uint64_t orc_max_encoded_size(uint64_t n, uint32_t B) {
  uint64_t nchunks = ceil_div(n, ORC_CHUNK);
  uint64_t size = payload_pos(nchunks);
  for (uint64_t c = 0; c < nchunks; c++) {
    uint64_t nc = (n - c * ORC_CHUNK < ORC_CHUNK) ? n - c * ORC_CHUNK : ORC_CHUNK;
    size += pad128(nc);
    uint64_t plane;
    if (B != 0) {
      uint64_t nb = ceil_div(nc, B);
      size += pad128(ceil_div(nb, 8));
      plane = nb * B / 8;
    } else {
      plane = ceil_div(nc, 8);
    }
    size += 3ull * pad128(plane);
    size += pad128(nc);
  }
  return size;
}

/* ---- 3-bit encode ------------------------------------------------------- */

/* Values in chunk c. */
static uint64_t chunk_len(uint64_t n, uint64_t c) {
  const uint64_t start = c * ORC_CHUNK;
  return (n - start < ORC_CHUNK) ? n - start : ORC_CHUNK;
}

/* What the writer of one chunk reads. */
typedef struct {
  const uint16_t* x;
  uint64_t n;
  uint32_t B;             /* 0: zip3 mode */
  const uint8_t* changed; /* ciera mode: one flag per block */
  unsigned e0;
  uint64_t nchunks;
  uint8_t* out;
} orc_enc;

/* Writes chunk c's table entry, its sections from stream offset pos and its
 * escape-index entry; returns the offset after its last section.  *nch_out
 * and *nesc_out receive its changed blocks and escapes. */
static uint64_t encode_chunk(const orc_enc* e, uint64_t c, uint64_t pos, uint64_t* nch_out, uint64_t* nesc_out) {
  const int ciera = (e->B != 0);
  const uint32_t B = e->B;
  const uint16_t* x = e->x;
  uint8_t* out = e->out;
  const uint64_t start = c * ORC_CHUNK;
  const uint64_t nc = chunk_len(e->n, c);
  put_u64(out + ORC_HEADER + 8ull * c, pos);
  /* escape index: escapes among the chunk's values before quarter q */
  uint64_t quarter_esc[4] = {0, 0, 0, 0};
  unsigned next_q = 1;

  /* 1. sign+mantissa bytes of every value */
  for (uint64_t t = 0; t < nc; t++) out[pos + t] = (uint8_t)sm_field(x[start + t]);
  pos += pad128(nc);

  /* 2. bitmap of changed blocks */
  uint64_t nch = 0, nb = 0;
  if (ciera) {
    nb = ceil_div(nc, B);
    for (uint64_t j = 0; j < nb; j++) {
      if (e->changed[start / B + j]) {
        out[pos + j / 8] |= (uint8_t)(1u << (j % 8));
        nch++;
      }
    }
    pos += pad128(ceil_div(nb, 8));
  }

  /* 3./4. code planes and escapes, slot by slot */
  const uint64_t plane_bytes = ciera ? nch * B / 8 : ceil_div(nc, 8);
  const uint64_t plane_pos[3] = {pos, pos + pad128(plane_bytes), pos + 2 * pad128(plane_bytes)};
  const uint64_t esc_pos = pos + 3 * pad128(plane_bytes);
  uint64_t nesc = 0;
  uint64_t slot = 0;
  if (!ciera) {
    for (uint64_t t = 0; t < nc; t++, slot++) {
      while (next_q < 4u && t >= next_q * ORC_QUARTER) quarter_esc[next_q++] = nesc;
      unsigned ex = exp_field(x[start + t]);
      unsigned code = code_of(ex, e->e0);
      for (int b = 0; b < 3; b++)
        if ((code >> b) & 1u) out[plane_pos[b] + slot / 8] |= (uint8_t)(1u << (slot % 8));
      if (code == 0) out[esc_pos + nesc++] = (uint8_t)ex;
    }
  } else {
    for (uint64_t j = 0; j < nb; j++) {
      if (!e->changed[start / B + j]) continue;
      for (uint64_t s = 0; s < B; s++, slot++) {
        uint64_t t = j * B + s;
        if (t >= nc) continue; /* slot past the end of the data: stays 0 */
        while (next_q < 4u && t >= next_q * ORC_QUARTER) quarter_esc[next_q++] = nesc;
        unsigned ex = exp_field(x[start + t]);
        unsigned code = code_of(ex, e->e0);
        for (int b = 0; b < 3; b++)
          if ((code >> b) & 1u) out[plane_pos[b] + slot / 8] |= (uint8_t)(1u << (slot % 8));
        if (code == 0) out[esc_pos + nesc++] = (uint8_t)ex;
      }
    }
  }
  while (next_q < 4u) quarter_esc[next_q++] = nesc;
  for (unsigned q = 0; q < 4u; q++)
    put_u16(out + index_pos(e->nchunks) + 8ull * c + 2ull * q, (unsigned)quarter_esc[q]);
  *nch_out = nch;
  *nesc_out = nesc;
  return esc_pos + pad128(nesc);
}

static void write_header(uint8_t* out, int ciera, unsigned e0, uint64_t n, uint32_t B, uint64_t nchunks,
                         uint64_t total, uint64_t changed, uint64_t esc) {
  put_u64(out + ORC_HEADER + 8ull * nchunks, total);
  memcpy(out, ciera ? "CIER" : "ZIP3", 4);
  put_u16(out + 4, 1);
  out[6] = (uint8_t)(ciera ? 1 : 0);
  out[7] = (uint8_t)e0;
  put_u64(out + 8, n);
  put_u32(out + 16, B);
  put_u32(out + 20, (uint32_t)ORC_CHUNK);
  put_u64(out + 24, nchunks);
  put_u64(out + 32, total);
  put_u64(out + 40, changed);
  put_u64(out + 48, esc);
}

static int check_encode_args(const uint16_t* x, uint64_t n, uint32_t B, const uint8_t* cache, int e0_override,
                             const uint8_t* out, uint64_t capacity) {
  if (n > ORC_MAX_N) return ORC_ERR_ARG;
  if (B != 0 && !valid_block_size(B)) return ORC_ERR_ARG;
  if (B != 0 && n > 0 && cache == NULL) return ORC_ERR_ARG;
  if (n > 0 && x == NULL) return ORC_ERR_ARG;
  if (e0_override < -1 || e0_override > 249) return ORC_ERR_ARG;
  if (out == NULL || capacity < orc_max_encoded_size(n, B)) return ORC_ERR_CAPACITY;
  return ORC_OK;
}

/* Encode.  B = 0: zip3 mode (every value coded, cache unused and may be
 * NULL).  B != 0: ciera mode; cache holds n exponent bytes from the previous
 * iteration (all zero before the first) and is overwritten with x's
 * exponents.  e0_override in [0, 249] forces the window base, -1 derives it
 * from the variance.  stats (may be NULL) receives {E0, changed blocks,
 * escapes}. */
int orc_encode(const uint16_t* x, uint64_t n, uint32_t B, uint8_t* cache, int e0_override,
               uint8_t* out, uint64_t capacity, uint64_t* out_size, uint64_t* stats) {
  const int ciera = (B != 0);
  int st = check_encode_args(x, n, B, cache, e0_override, out, capacity);
  if (st != ORC_OK) return st;
  memset(out, 0, orc_max_encoded_size(n, B));

  const unsigned e0 = (e0_override >= 0) ? (unsigned)e0_override : (unsigned)orc_choose_e0(x, n);
  const uint64_t nchunks = ceil_div(n, ORC_CHUNK);

  /* Block change flags against the sender cache. */
  uint8_t* changed = NULL;
  if (ciera) {
    changed = (uint8_t*)calloc(ceil_div(n, B) + 1u, 1);
    if (!changed) return ORC_ERR_NOMEM;
    for (uint64_t i = 0; i < n; i++) {
      if (exp_field(x[i]) != cache[i]) changed[i / B] = 1;
    }
  }

  const orc_enc e = {x, n, B, changed, e0, nchunks, out};
  uint64_t pos = payload_pos(nchunks);
  uint64_t total_changed = 0, total_esc = 0;
  for (uint64_t c = 0; c < nchunks; c++) {
    uint64_t nch, nesc;
    pos = encode_chunk(&e, c, pos, &nch, &nesc);
    total_changed += nch;
    total_esc += nesc;
  }
  write_header(out, ciera, e0, n, B, nchunks, pos, total_changed, total_esc);

  if (ciera) {
    for (uint64_t i = 0; i < n; i++) cache[i] = (uint8_t)exp_field(x[i]);
    free(changed);
  }
  *out_size = pos;
  if (stats) {
    stats[0] = e0;
    stats[1] = total_changed;
    stats[2] = total_esc;
  }
  return ORC_OK;
}

/* ---- 3-bit decode ------------------------------------------------------- */

/* Checks the header and the table's first and last entries. */
static int check_stream_header(const uint8_t* in, uint64_t in_size, uint64_t n, uint32_t B, unsigned* e0_out,
                               uint64_t* total_out) {
  const int ciera = (B != 0);
  if (in == NULL || in_size < ORC_HEADER) return ORC_ERR_FORMAT;
  const uint64_t nchunks = ceil_div(n, ORC_CHUNK);
  const uint64_t base = payload_pos(nchunks);
  if (memcmp(in, ciera ? "CIER" : "ZIP3", 4) != 0) return ORC_ERR_FORMAT;
  if (get_u16(in + 4) != 1u) return ORC_ERR_FORMAT;
  if (in[6] != (ciera ? 1 : 0)) return ORC_ERR_FORMAT;
  const unsigned e0 = in[7];
  if (e0 > 249u) return ORC_ERR_FORMAT;
  if (get_u64(in + 8) != n) return ORC_ERR_FORMAT;
  if (get_u32(in + 16) != B) return ORC_ERR_FORMAT;
  if (get_u32(in + 20) != (uint32_t)ORC_CHUNK) return ORC_ERR_FORMAT;
  if (get_u64(in + 24) != nchunks) return ORC_ERR_FORMAT;
  const uint64_t total = get_u64(in + 32);
  if (total > in_size || base > in_size) return ORC_ERR_FORMAT;
  for (uint64_t i = 56; i < ORC_HEADER; i++)
    if (in[i] != 0) return ORC_ERR_FORMAT;
  if (get_u64(in + ORC_HEADER) != base) return ORC_ERR_FORMAT;
  if (get_u64(in + ORC_HEADER + 8ull * nchunks) != total) return ORC_ERR_FORMAT;
  for (uint64_t i = index_pos(nchunks) + 8ull * nchunks; i < base; i++)
    if (in[i] != 0) return ORC_ERR_FORMAT;
  *e0_out = e0;
  *total_out = total;
  return ORC_OK;
}

/* Decodes chunk c of a stream whose header passed check_stream_header:
 * writes its values to y (and, ciera, the changed blocks' exponents to
 * cache) and returns ORC_OK with its changed blocks and escapes, or
 * ORC_ERR_FORMAT when its sections or escape-index entry do not match. */
static int decode_chunk(const uint8_t* in, uint64_t n, uint32_t B, unsigned e0, uint64_t total, uint64_t c,
                        uint16_t* y, uint8_t* cache, uint64_t* nch_out, uint64_t* nesc_out) {
  const int ciera = (B != 0);
  const uint64_t nchunks = ceil_div(n, ORC_CHUNK);
  const uint64_t start = c * ORC_CHUNK;
  const uint64_t nc = chunk_len(n, c);
  const uint64_t begin = get_u64(in + ORC_HEADER + 8ull * c);
  const uint64_t end = get_u64(in + ORC_HEADER + 8ull * (c + 1));
  if (begin > end || end > total) return ORC_ERR_FORMAT;

  uint64_t pos = begin;
  const uint64_t sm_pos = pos;
  pos += pad128(nc);
  uint64_t bitmap_pos = 0, nb = 0, nch = 0;
  if (ciera) {
    nb = ceil_div(nc, B);
    bitmap_pos = pos;
    pos += pad128(ceil_div(nb, 8));
    if (pos > end) return ORC_ERR_FORMAT;
    for (uint64_t j = 0; j < nb; j++) nch += (in[bitmap_pos + j / 8] >> (j % 8)) & 1u;
  }
  const uint64_t plane_bytes = ciera ? nch * B / 8 : ceil_div(nc, 8);
  const uint64_t plane_pos[3] = {pos, pos + pad128(plane_bytes), pos + 2 * pad128(plane_bytes)};
  const uint64_t esc_pos = pos + 3 * pad128(plane_bytes);
  if (esc_pos > end) return ORC_ERR_FORMAT;

  uint64_t nesc = 0;
  uint64_t quarter_esc[4] = {0, 0, 0, 0};
  unsigned next_q = 1;
  if (!ciera) {
    for (uint64_t t = 0; t < nc; t++) {
      while (next_q < 4u && t >= next_q * ORC_QUARTER) quarter_esc[next_q++] = nesc;
      unsigned code = 0, e;
      for (int b = 0; b < 3; b++) code |= ((in[plane_pos[b] + t / 8] >> (t % 8)) & 1u) << b;
      if (code != 0) {
        e = e0 + code - 1u;
      } else {
        if (esc_pos + nesc >= end) return ORC_ERR_FORMAT;
        e = in[esc_pos + nesc++];
      }
      y[start + t] = join_fields(in[sm_pos + t], e);
    }
  } else {
    uint64_t rank = 0; /* changed blocks of this chunk seen so far */
    for (uint64_t j = 0; j < nb; j++) {
      const int is_changed = (in[bitmap_pos + j / 8] >> (j % 8)) & 1u;
      for (uint64_t s = 0; s < B && j * B + s < nc; s++) {
        const uint64_t t = j * B + s;
        while (next_q < 4u && t >= next_q * ORC_QUARTER) quarter_esc[next_q++] = nesc;
        unsigned e;
        if (!is_changed) {
          e = cache[start + t];
        } else {
          const uint64_t slot = rank * B + s;
          unsigned code = 0;
          for (int b = 0; b < 3; b++)
            code |= ((in[plane_pos[b] + slot / 8] >> (slot % 8)) & 1u) << b;
          if (code != 0) {
            e = e0 + code - 1u;
          } else {
            if (esc_pos + nesc >= end) return ORC_ERR_FORMAT;
            e = in[esc_pos + nesc++];
          }
          cache[start + t] = (uint8_t)e;
        }
        y[start + t] = join_fields(in[sm_pos + t], e);
      }
      if (is_changed) rank++;
    }
  }
  if (esc_pos + pad128(nesc) != end) return ORC_ERR_FORMAT;
  while (next_q < 4u) quarter_esc[next_q++] = nesc;
  for (unsigned q = 0; q < 4u; q++)
    if (get_u16(in + index_pos(nchunks) + 8ull * c + 2ull * q) != quarter_esc[q]) return ORC_ERR_FORMAT;
  *nch_out = nch;
  *nesc_out = nesc;
  return ORC_OK;
}

static int check_decode_args(uint64_t n, uint32_t B, const uint16_t* y, const uint8_t* cache) {
  if (n > ORC_MAX_N) return ORC_ERR_ARG;
  if (B != 0 && !valid_block_size(B)) return ORC_ERR_ARG;
  if (n > 0 && (y == NULL || (B != 0 && cache == NULL))) return ORC_ERR_ARG;
  return ORC_OK;
}

/* Decode.  B = 0 expects a zip3 stream; B != 0 a ciera stream with that B,
 * and cache holds the receiver's exponents of the previous iteration (updated
 * in place).  Every header field, table entry and section size is checked
 * against the layout above; any mismatch returns ORC_ERR_FORMAT.  in_size
 * may exceed the stream's total_bytes (the rest is not read). */
int orc_decode(const uint8_t* in, uint64_t in_size, uint16_t* y, uint64_t n, uint32_t B,
               uint8_t* cache) {
  int st = check_decode_args(n, B, y, cache);
  if (st != ORC_OK) return st;
  unsigned e0;
  uint64_t total;
  st = check_stream_header(in, in_size, n, B, &e0, &total);
  if (st != ORC_OK) return st;
  const uint64_t nchunks = ceil_div(n, ORC_CHUNK);
  uint64_t total_changed = 0, total_esc = 0;
  for (uint64_t c = 0; c < nchunks; c++) {
    uint64_t nch, nesc;
    st = decode_chunk(in, n, B, e0, total, c, y, cache, &nch, &nesc);
    if (st != ORC_OK) return st;
    total_changed += nch;
    total_esc += nesc;
  }
  if (get_u64(in + 40) != total_changed || get_u64(in + 48) != total_esc) return ORC_ERR_FORMAT;
  return ORC_OK;
}

/* ---- chunk-parallel drivers --------------------------------------------- */

#define ORC_MAX_THREADS 256

typedef void (*orc_range_fn)(void* arg, int job, uint64_t begin, uint64_t end);
typedef struct {
  orc_range_fn fn;
  void* arg;
  int job;
  uint64_t begin, end;
} orc_job;

static void* job_main(void* p) {
  orc_job* j = (orc_job*)p;
  j->fn(j->arg, j->job, j->begin, j->end);
  return NULL;
}

/* Runs fn over [0, count) split into `jobs` contiguous ranges, one thread
 * each (a thread that cannot be created runs its range on the caller). */
static void parallel_for(int jobs, uint64_t count, orc_range_fn fn, void* arg) {
  pthread_t th[ORC_MAX_THREADS];
  orc_job job[ORC_MAX_THREADS];
  int started[ORC_MAX_THREADS];
  for (int t = 0; t < jobs; t++) {
    job[t].fn = fn;
    job[t].arg = arg;
    job[t].job = t;
    job[t].begin = count * (uint64_t)t / (uint64_t)jobs;
    job[t].end = count * (uint64_t)(t + 1) / (uint64_t)jobs;
    started[t] = (t > 0) && pthread_create(&th[t], NULL, job_main, &job[t]) == 0;
  }
  for (int t = 0; t < jobs; t++)
    if (!started[t]) job_main(&job[t]);
  for (int t = 1; t < jobs; t++)
    if (started[t]) pthread_join(th[t], NULL);
}

static int clamp_threads(int nthreads) {
  if (nthreads < 1) return 1;
  return nthreads > ORC_MAX_THREADS ? ORC_MAX_THREADS : nthreads;
}

typedef struct {
  const uint16_t* x;
  uint64_t n;
  uint32_t B;
  uint8_t* cache;
  uint8_t* changed;
  uint8_t* out;
  orc_enc enc;
  int64_t (*a)[256];
  uint64_t (*b)[256];
  uint64_t* nf;
  uint64_t* nch;  /* per chunk */
  uint64_t* nesc; /* per chunk */
  uint64_t* off;  /* per chunk + 1 */
  int bad;        /* a chunk's writer ended off its closed-form size */
} orc_mt;

static void mt_zero(void* p, int job, uint64_t begin, uint64_t end) {
  (void)job;
  memset(((orc_mt*)p)->out + begin, 0, end - begin);
}

static void mt_sums(void* p, int job, uint64_t begin, uint64_t end) {
  orc_mt* m = (orc_mt*)p;
  orc_exponent_sums(m->x + begin, end - begin, m->a[job], m->b[job], &m->nf[job]);
}

static void mt_changed(void* p, int job, uint64_t begin, uint64_t end) {
  (void)job;
  orc_mt* m = (orc_mt*)p;
  for (uint64_t blk = begin; blk < end; blk++) {
    const uint64_t i_end = (blk + 1) * m->B < m->n ? (blk + 1) * m->B : m->n;
    for (uint64_t i = blk * m->B; i < i_end; i++)
      if (exp_field(m->x[i]) != m->cache[i]) {
        m->changed[blk] = 1;
        break;
      }
  }
}

/* Changed blocks and escapes of each chunk, counted value by value. */
static void mt_counts(void* p, int job, uint64_t begin, uint64_t end) {
  (void)job;
  orc_mt* m = (orc_mt*)p;
  for (uint64_t c = begin; c < end; c++) {
    const uint64_t start = c * ORC_CHUNK, nc = chunk_len(m->n, c);
    uint64_t nch = 0, nesc = 0;
    if (m->B)
      for (uint64_t j = 0; j < ceil_div(nc, m->B); j++) nch += m->changed[start / m->B + j];
    for (uint64_t t = 0; t < nc; t++) {
      const int coded = (m->B == 0) || m->changed[(start + t) / m->B];
      if (coded && code_of(exp_field(m->x[start + t]), m->enc.e0) == 0) nesc++;
    }
    m->nch[c] = nch;
    m->nesc[c] = nesc;
  }
}

static void mt_write(void* p, int job, uint64_t begin, uint64_t end) {
  (void)job;
  orc_mt* m = (orc_mt*)p;
  for (uint64_t c = begin; c < end; c++) {
    uint64_t nch, nesc;
    const uint64_t after = encode_chunk(&m->enc, c, m->off[c], &nch, &nesc);
    if (after != m->off[c + 1] || nch != m->nch[c] || nesc != m->nesc[c]) m->bad = 1;
  }
}

static void mt_cache(void* p, int job, uint64_t begin, uint64_t end) {
  (void)job;
  orc_mt* m = (orc_mt*)p;
  for (uint64_t i = begin; i < end; i++) m->cache[i] = (uint8_t)exp_field(m->x[i]);
}

/* Stream bytes of a chunk of nc values with nch changed blocks (ciera) and
 * nesc escapes: the sections' padded sizes added up. */
static uint64_t chunk_bytes(uint64_t nc, uint32_t B, uint64_t nch, uint64_t nesc) {
  uint64_t s = pad128(nc), plane;
  if (B != 0) {
    s += pad128(ceil_div(ceil_div(nc, B), 8));
    plane = nch * B / 8;
  } else {
    plane = ceil_div(nc, 8);
  }
  return s + 3ull * pad128(plane) + pad128(nesc);
}

/* orc_encode on nthreads threads: the same window (exact integer sums added
 * across threads), change flags, per-chunk writer and header, so the stream
 * and the cache are byte-equal to orc_encode's.  Chunk offsets come from the
 * chunks' counts through chunk_bytes; a chunk whose writer ends elsewhere
 * makes the call fail with ORC_ERR_INTERNAL. */
#define ORC_ERR_INTERNAL 7
int orc_encode_mt(const uint16_t* x, uint64_t n, uint32_t B, uint8_t* cache, int e0_override, uint8_t* out,
                  uint64_t capacity, uint64_t* out_size, uint64_t* stats, int nthreads) {
  const int ciera = (B != 0);
  int st = check_encode_args(x, n, B, cache, e0_override, out, capacity);
  if (st != ORC_OK) return st;
  const int T = clamp_threads(nthreads);
  const uint64_t nchunks = ceil_div(n, ORC_CHUNK);
  orc_mt m;
  memset(&m, 0, sizeof(m));
  m.x = x;
  m.n = n;
  m.B = B;
  m.cache = cache;
  m.out = out;
  m.a = (int64_t(*)[256])calloc((size_t)T, sizeof(*m.a));
  m.b = (uint64_t(*)[256])calloc((size_t)T, sizeof(*m.b));
  m.nf = (uint64_t*)calloc((size_t)T, sizeof(uint64_t));
  m.nch = (uint64_t*)calloc(nchunks + 1u, sizeof(uint64_t));
  m.nesc = (uint64_t*)calloc(nchunks + 1u, sizeof(uint64_t));
  m.off = (uint64_t*)calloc(nchunks + 1u, sizeof(uint64_t));
  m.changed = ciera ? (uint8_t*)calloc(ceil_div(n, B) + 1u, 1) : NULL;
  if (!m.a || !m.b || !m.nf || !m.nch || !m.nesc || !m.off || (ciera && !m.changed)) {
    st = ORC_ERR_NOMEM;
    goto done;
  }
  parallel_for(T, orc_max_encoded_size(n, B), mt_zero, &m);

  unsigned e0;
  if (e0_override >= 0) {
    e0 = (unsigned)e0_override;
  } else {
    parallel_for(T, n, mt_sums, &m);
    int64_t a[256] = {0};
    uint64_t b[256] = {0}, nf = 0;
    for (int t = 0; t < T; t++) {
      for (unsigned k = 0; k < 256u; k++) {
        a[k] += m.a[t][k];
        b[k] += m.b[t][k];
      }
      nf += m.nf[t];
    }
    e0 = (unsigned)orc_window_base_exact(a, b, nf);
  }
  if (ciera) parallel_for(T, ceil_div(n, B), mt_changed, &m);
  const orc_enc e = {x, n, B, m.changed, e0, nchunks, out};
  m.enc = e;
  parallel_for(T, nchunks, mt_counts, &m);
  uint64_t total_changed = 0, total_esc = 0;
  m.off[0] = payload_pos(nchunks);
  for (uint64_t c = 0; c < nchunks; c++) {
    m.off[c + 1] = m.off[c] + chunk_bytes(chunk_len(n, c), B, m.nch[c], m.nesc[c]);
    total_changed += m.nch[c];
    total_esc += m.nesc[c];
  }
  parallel_for(T, nchunks, mt_write, &m);
  if (m.bad) {
    st = ORC_ERR_INTERNAL;
    goto done;
  }
  write_header(out, ciera, e0, n, B, nchunks, m.off[nchunks], total_changed, total_esc);
  if (ciera) parallel_for(T, n, mt_cache, &m);
  *out_size = m.off[nchunks];
  if (stats) {
    stats[0] = e0;
    stats[1] = total_changed;
    stats[2] = total_esc;
  }
done:
  free(m.a);
  free(m.b);
  free(m.nf);
  free(m.nch);
  free(m.nesc);
  free(m.off);
  free(m.changed);
  return st;
}

typedef struct {
  const uint8_t* in;
  uint64_t n;
  uint32_t B;
  unsigned e0;
  uint64_t total;
  uint16_t* y;
  uint8_t* cache;
  int* status;    /* per job */
  uint64_t* nch;  /* per job */
  uint64_t* nesc; /* per job */
} orc_mt_dec;

static void mt_decode(void* p, int job, uint64_t begin, uint64_t end) {
  orc_mt_dec* d = (orc_mt_dec*)p;
  uint64_t nch_sum = 0, nesc_sum = 0;
  int st = ORC_OK;
  for (uint64_t c = begin; c < end && st == ORC_OK; c++) {
    uint64_t nch, nesc;
    st = decode_chunk(d->in, d->n, d->B, d->e0, d->total, c, d->y, d->cache, &nch, &nesc);
    nch_sum += nch;
    nesc_sum += nesc;
  }
  d->status[job] = st;
  d->nch[job] = nch_sum;
  d->nesc[job] = nesc_sum;
}

/* orc_decode on nthreads threads (chunks are decoded by the same per-chunk
 * step; the same checks, the same result). */
int orc_decode_mt(const uint8_t* in, uint64_t in_size, uint16_t* y, uint64_t n, uint32_t B, uint8_t* cache,
                  int nthreads) {
  int st = check_decode_args(n, B, y, cache);
  if (st != ORC_OK) return st;
  orc_mt_dec d;
  memset(&d, 0, sizeof(d));
  st = check_stream_header(in, in_size, n, B, &d.e0, &d.total);
  if (st != ORC_OK) return st;
  const int T = clamp_threads(nthreads);
  d.in = in;
  d.n = n;
  d.B = B;
  d.y = y;
  d.cache = cache;
  d.status = (int*)calloc((size_t)T, sizeof(int));
  d.nch = (uint64_t*)calloc((size_t)T, sizeof(uint64_t));
  d.nesc = (uint64_t*)calloc((size_t)T, sizeof(uint64_t));
  if (!d.status || !d.nch || !d.nesc) {
    st = ORC_ERR_NOMEM;
  } else {
    parallel_for(T, ceil_div(n, ORC_CHUNK), mt_decode, &d);
    uint64_t total_changed = 0, total_esc = 0;
    for (int t = 0; t < T; t++) {
      if (d.status[t] != ORC_OK) st = d.status[t];
      total_changed += d.nch[t];
      total_esc += d.nesc[t];
    }
    if (st == ORC_OK && (get_u64(in + 40) != total_changed || get_u64(in + 48) != total_esc)) st = ORC_ERR_FORMAT;
  }
  free(d.status);
  free(d.nch);
  free(d.nesc);
  return st;
}

/* ------------------------------------------------------------------------
 * rANS variant (modes 2 = zip3 + rANS, 3 = ciera + rANS).  The coded
 * exponents (all of them in zip3 mode, those of changed blocks in ciera mode)
 * are entropy coded with range ANS instead of the 3-bit window code, in
 * place of the ANS coder the CIERA page uses for changed exponents (section
 * 3.1: the sender ANS-encodes the changed exponents, the receiver
 * ANS-decodes them).  The page names no ANS parameters; this format is ours.
 *
 *  - Symbols: the exponent fields of a chunk's coded values.  Part h of the
 *    chunk (values [16384 h, 16384 (h+1)) of it) holds the coded ones among
 *    its values, in value order: s_0 .. s_{m_h - 1}.
 *  - Frequencies: one table per chunk, from the histogram h over all of its
 *    m = m_0 + m_1 + m_2 + m_3 symbols, normalised to M = 4096: with d
 *    distinct symbols, f_s = max(1, floor(h_s (M - d) / m)) for every
 *    symbol present (0 otherwise), and the rest, M - sum f, is added to the
 *    most frequent symbol (the lowest one on ties).  c_s is the sum of f
 *    over the symbols below s.
 *  - Coding: each part codes its own symbols with the chunk's table and 64
 *    interleaved rANS states; symbol i of the part goes to state i mod 64
 *    (step i div 64).  A state is a 32-bit x in [2^16, 2^32), starting at
 *    2^16.  Encoding runs over the steps from last to first; a state about
 *    to code symbol s first emits its low 16 bits and shifts right by 16
 *    when x >= f_s 2^20, then becomes (x div f_s) 2^12 + (x mod f_s) + c_s.
 *    Decoding runs forward: slot = x mod 2^12, s is the symbol whose range
 *    [c_s, c_s + f_s) holds slot, x becomes f_s (x div 2^12) + slot - c_s,
 *    and a state below 2^16 reads one 16-bit word: x = x 2^16 + word.
 *  - Chunk payload (little-endian): u8 lo, u8 hi (the first and last symbol
 *    with f > 0), u16 0, u16 w_0 .. w_3 (the number of 16-bit words in each
 *    part's stream), f_lo .. f_hi as u16, then the four part streams in
 *    part order.  A part's stream: the 64 final encoder states (low half,
 *    high half, state 0 first), then, step by step from the first, the
 *    words the encoder emitted at that step, in ascending state order; a
 *    part without coded symbols has an empty stream (w_h = 0).  A chunk
 *    without coded symbols has an empty payload.
 *  - Stream: the 128-byte header (version 2, mode 2 or 3, E0 = 0, bytes
 *    48..55 the number of coded symbols); at byte 128 a chunk table of
 *    nchunks + 1 u64 absolute payload offsets (the last is total_bytes),
 *    zero-padded to 128; then the sign+mantissa bytes of all n values,
 *    zero-padded to 128; in ciera mode the chunks' bitmaps, 128 bytes each
 *    (bit j & 7 of byte j >> 3 for block j of the chunk); then the chunk
 *    payloads, each zero-padded to 128.
 * A decoder checks that every word is used and that every state ends at
 * 2^16, the encoder's start.
 * ------------------------------------------------------------------------ */
#define ORC_RANS_M 4096u
#define ORC_RANS_L 65536u
#define ORC_RANS_LANES 64u
#define ORC_PART 16384ull
#define ORC_RANS_HEAD 12ull
#define ORC_RANS_VERSION 2u

void orc_rans_freqs(const uint32_t hist[256], uint16_t freq[256]) {
  uint64_t m = 0;
  unsigned d = 0, top = 0;
  for (unsigned s = 0; s < 256; s++) {
    m += hist[s];
    if (hist[s]) d++;
    if (hist[s] > hist[top]) top = s;
  }
  if (m == 0) {
    memset(freq, 0, 256 * sizeof(uint16_t));
    return;
  }
  unsigned sum = 0;
  for (unsigned s = 0; s < 256; s++) {
    unsigned f = 0;
    if (hist[s]) {
      f = (unsigned)((uint64_t)hist[s] * (ORC_RANS_M - d) / m);
      if (f == 0) f = 1;
    }
    freq[s] = (uint16_t)f;
    sum += f;
  }
  freq[top] = (uint16_t)(freq[top] + (ORC_RANS_M - sum));
}

/* Largest payload of a chunk of nc values: every value coded, and at most
 * one word emitted per symbol. */
static uint64_t rans_chunk_max(uint64_t nc) {
  if (nc == 0) return 0;
  return ORC_RANS_HEAD + 512ull + 2ull * (2ull * ORC_RANS_LANES * ceil_div(nc, ORC_PART) + nc);
}

uint64_t orc_rans_max_encoded_size(uint64_t n, uint32_t B) {
  uint64_t nchunks = ceil_div(n, ORC_CHUNK);
  uint64_t size = ORC_HEADER + pad128(8ull * (nchunks + 1ull)) + pad128(n);
  if (B) size += 128ull * nchunks;
  for (uint64_t v = 0; v < n; v += ORC_CHUNK) size += pad128(rans_chunk_max((n - v < ORC_CHUNK) ? n - v : ORC_CHUNK));
  return size;
}

/* One part's stream: its m symbols coded with the chunk's table (f, cum),
 * written at out.  Returns its number of 16-bit words (0 for m = 0). */
static uint64_t rans_encode_stream(const uint8_t* sym, uint64_t m, const uint16_t* f, const uint32_t* cum,
                                   uint8_t* out) {
  if (m == 0) return 0;
  const uint64_t steps = ceil_div(m, ORC_RANS_LANES);
  uint32_t x[ORC_RANS_LANES];
  for (unsigned l = 0; l < ORC_RANS_LANES; l++) x[l] = ORC_RANS_L;
  /* emitted words in encode order (last step first) and each step's count */
  uint16_t* emit = (uint16_t*)malloc(m * sizeof(uint16_t));
  uint64_t* count = (uint64_t*)calloc(steps, sizeof(uint64_t));
  uint64_t ne = 0;
  for (uint64_t t = steps; t-- > 0;) {
    for (unsigned l = 0; l < ORC_RANS_LANES; l++) {
      uint64_t i = t * ORC_RANS_LANES + l;
      if (i >= m) break;
      unsigned s = sym[i];
      uint64_t xmax = (uint64_t)f[s] << 20;
      if (x[l] >= xmax) {
        emit[ne++] = (uint16_t)(x[l] & 0xFFFFu);
        count[t]++;
        x[l] >>= 16;
      }
      x[l] = (x[l] / f[s]) * ORC_RANS_M + (x[l] % f[s]) + cum[s];
    }
  }
  uint8_t* p = out;
  for (unsigned l = 0; l < ORC_RANS_LANES; l++, p += 4) {
    put_u16(p, x[l] & 0xFFFFu);
    put_u16(p + 2, x[l] >> 16);
  }
  /* step t's words sit in emit[] after those of the steps above t */
  uint64_t above = 0;
  for (uint64_t t = steps; t-- > 0;) {
    uint64_t tmp = count[t];
    count[t] = above; /* now: index in emit[] of step t's first word */
    above += tmp;
  }
  for (uint64_t t = 0; t < steps; t++) {
    uint64_t first = count[t];
    uint64_t end = (t == 0) ? ne : count[t - 1];
    for (uint64_t k = first; k < end; k++, p += 2) put_u16(p, emit[k]);
  }
  free(emit);
  free(count);
  return 2ull * ORC_RANS_LANES + ne;
}

/* Payload of one chunk; sym holds the parts' symbols back to back, m[h] of
 * part h.  Returns its length in bytes (0 without symbols). */
static uint64_t rans_encode_chunk(const uint8_t* sym, const uint64_t m[4], uint8_t* out) {
  const uint64_t total = m[0] + m[1] + m[2] + m[3];
  if (total == 0) return 0;
  uint32_t hist[256] = {0};
  for (uint64_t i = 0; i < total; i++) hist[sym[i]]++;
  uint16_t f[256];
  orc_rans_freqs(hist, f);
  uint32_t cum[256];
  unsigned lo = 256, hi = 0, c = 0;
  for (unsigned s = 0; s < 256; s++) {
    cum[s] = c;
    c += f[s];
    if (f[s]) {
      if (lo == 256) lo = s;
      hi = s;
    }
  }
  out[0] = (uint8_t)lo;
  out[1] = (uint8_t)hi;
  out[2] = out[3] = 0;
  uint8_t* p = out + ORC_RANS_HEAD;
  for (unsigned s = lo; s <= hi; s++, p += 2) put_u16(p, f[s]);
  const uint8_t* s = sym;
  for (unsigned h = 0; h < 4; h++) {
    uint64_t w = rans_encode_stream(s, m[h], f, cum, p);
    put_u16(out + 4 + 2 * h, (unsigned)w);
    p += 2 * w;
    s += m[h];
  }
  return (uint64_t)(p - out);
}

/* Decode one part's stream (nwords words at w) into m symbols with the
 * chunk's table. */
static int rans_decode_stream(const uint8_t* w, uint64_t nwords, uint64_t m, const uint32_t* f, const uint32_t* cum,
                              const uint8_t* sym_of, uint8_t* sym) {
  if (m == 0) return nwords == 0 ? ORC_OK : ORC_ERR_FORMAT;
  if (nwords < 2ull * ORC_RANS_LANES) return ORC_ERR_FORMAT;
  uint32_t x[ORC_RANS_LANES];
  for (unsigned l = 0; l < ORC_RANS_LANES; l++) {
    x[l] = (uint32_t)get_u16(w + 4 * l) | ((uint32_t)get_u16(w + 4 * l + 2) << 16);
    if (x[l] < ORC_RANS_L) return ORC_ERR_FORMAT;
  }
  uint64_t q = 2ull * ORC_RANS_LANES;
  const uint64_t steps = ceil_div(m, ORC_RANS_LANES);
  for (uint64_t t = 0; t < steps; t++) {
    for (unsigned l = 0; l < ORC_RANS_LANES; l++) {
      uint64_t i = t * ORC_RANS_LANES + l;
      if (i >= m) break;
      unsigned slot = x[l] & (ORC_RANS_M - 1u);
      unsigned s = sym_of[slot];
      x[l] = f[s] * (x[l] >> 12) + slot - cum[s];
      if (x[l] < ORC_RANS_L) {
        if (q >= nwords) return ORC_ERR_FORMAT;
        x[l] = (x[l] << 16) | get_u16(w + 2 * q);
        q++;
      }
      sym[i] = (uint8_t)s;
    }
  }
  if (q != nwords) return ORC_ERR_FORMAT;
  for (unsigned l = 0; l < ORC_RANS_LANES; l++)
    if (x[l] != ORC_RANS_L) return ORC_ERR_FORMAT;
  return ORC_OK;
}

/* Decode one chunk's payload (len bytes, the padding excluded) into the
 * parts' symbols, back to back (m[h] of part h). */
static int rans_decode_chunk(const uint8_t* in, uint64_t len, const uint64_t m[4], uint8_t* sym) {
  if (len < ORC_RANS_HEAD) return ORC_ERR_FORMAT;
  unsigned lo = in[0], hi = in[1];
  if (hi < lo || in[2] || in[3]) return ORC_ERR_FORMAT;
  uint64_t nw[4], words = 0;
  for (unsigned h = 0; h < 4; h++) {
    nw[h] = get_u16(in + 4 + 2 * h);
    words += nw[h];
  }
  const uint64_t fbytes = 2ull * (hi - lo + 1u);
  if (len != ORC_RANS_HEAD + fbytes + 2 * words) return ORC_ERR_FORMAT;
  uint32_t f[256] = {0}, cum[256];
  unsigned total = 0;
  for (unsigned s = lo; s <= hi; s++) {
    f[s] = get_u16(in + ORC_RANS_HEAD + 2 * (s - lo));
    total += f[s];
  }
  if (total != ORC_RANS_M) return ORC_ERR_FORMAT;
  uint8_t sym_of[ORC_RANS_M];
  unsigned c = 0;
  for (unsigned s = 0; s < 256; s++) {
    cum[s] = c;
    for (unsigned k = 0; k < f[s]; k++) sym_of[c + k] = (uint8_t)s;
    c += f[s];
  }
  const uint8_t* p = in + ORC_RANS_HEAD + fbytes;
  for (unsigned h = 0; h < 4; h++) {
    int st = rans_decode_stream(p, nw[h], m[h], f, cum, sym_of, sym);
    if (st != ORC_OK) return st;
    p += 2 * nw[h];
    sym += m[h];
  }
  return ORC_OK;
}

static uint64_t rans_sm_pos(uint64_t nchunks) { return ORC_HEADER + pad128(8ull * (nchunks + 1ull)); }

/* Is value i coded?  zip3: always; ciera: when its block changed. */
static int rans_coded(const uint8_t* changed, uint32_t B, uint64_t i) { return B == 0 || changed[i / B]; }

/* Is value i coded, by the stream's bitmap (ciera; zip3: always)? */
static int rans_bit(const uint8_t* in, uint64_t bm_pos, uint32_t B, uint64_t i) {
  if (B == 0) return 1;
  uint64_t c = i / ORC_CHUNK, j = (i % ORC_CHUNK) / B;
  return (in[bm_pos + 128 * c + (j >> 3)] >> (j & 7)) & 1;
}

/* Encode in an rANS mode (B = 0: zip3 + rANS; else ciera + rANS with the
 * sender cache as in orc_encode).  stats (may be NULL): {changed blocks,
 * coded symbols}. */
int orc_encode_rans(const uint16_t* x, uint64_t n, uint32_t B, uint8_t* cache, uint8_t* out, uint64_t capacity,
                    uint64_t* out_size, uint64_t* stats) {
  const int ciera = (B != 0);
  if (n > ORC_MAX_N) return ORC_ERR_ARG;
  if (ciera && !valid_block_size(B)) return ORC_ERR_ARG;
  if (ciera && n > 0 && cache == NULL) return ORC_ERR_ARG;
  if (n > 0 && x == NULL) return ORC_ERR_ARG;
  const uint64_t need = orc_rans_max_encoded_size(n, B);
  if (out == NULL || capacity < need) return ORC_ERR_CAPACITY;
  memset(out, 0, need);
  const uint64_t nchunks = ceil_div(n, ORC_CHUNK);
  const uint64_t nblocks = ciera ? ceil_div(n, B) : 0;
  uint8_t* changed = NULL;
  uint64_t n_changed = 0;
  if (ciera) {
    changed = (uint8_t*)calloc(nblocks ? nblocks : 1, 1);
    if (!changed) return ORC_ERR_NOMEM;
    for (uint64_t i = 0; i < n; i++)
      if (exp_field(x[i]) != cache[i]) changed[i / B] = 1;
    for (uint64_t b = 0; b < nblocks; b++) n_changed += changed[b];
  }
  const uint64_t sm_pos = rans_sm_pos(nchunks);
  const uint64_t bm_pos = sm_pos + pad128(n);
  uint64_t pos = bm_pos + (ciera ? 128ull * nchunks : 0);
  for (uint64_t i = 0; i < n; i++) out[sm_pos + i] = (uint8_t)sm_field(x[i]);
  if (ciera) {
    for (uint64_t c = 0; c < nchunks; c++)
      for (uint64_t j = 0; j < ORC_CHUNK / B && c * ORC_CHUNK + j * B < n; j++)
        if (changed[c * (ORC_CHUNK / B) + j]) out[bm_pos + 128 * c + (j >> 3)] |= (uint8_t)(1u << (j & 7));
  }
  uint8_t* sym = (uint8_t*)malloc(ORC_CHUNK);
  uint64_t n_coded = 0;
  for (uint64_t c = 0; c < nchunks; c++) {
    put_u64(out + ORC_HEADER + 8 * c, pos);
    uint64_t m[4], k = 0;
    for (unsigned h = 0; h < 4; h++) {
      uint64_t begin = c * ORC_CHUNK + h * ORC_PART;
      uint64_t end = begin + ORC_PART < n ? begin + ORC_PART : n;
      m[h] = 0;
      for (uint64_t i = begin; i < end; i++)
        if (rans_coded(changed, B, i)) {
          sym[k++] = (uint8_t)exp_field(x[i]);
          m[h]++;
        }
    }
    n_coded += k;
    pos += pad128(rans_encode_chunk(sym, m, out + pos));
  }
  free(sym);
  put_u64(out + ORC_HEADER + 8 * nchunks, pos);
  memcpy(out, ciera ? "CIER" : "ZIP3", 4);
  put_u16(out + 4, ORC_RANS_VERSION);
  out[6] = ciera ? 3 : 2;
  out[7] = 0;
  put_u64(out + 8, n);
  put_u32(out + 16, B);
  put_u32(out + 20, (uint32_t)ORC_CHUNK);
  put_u64(out + 24, nchunks);
  put_u64(out + 32, pos);
  put_u64(out + 40, n_changed);
  put_u64(out + 48, n_coded);
  if (ciera)
    for (uint64_t i = 0; i < n; i++) cache[i] = (uint8_t)exp_field(x[i]);
  free(changed);
  *out_size = pos;
  if (stats) {
    stats[0] = n_changed;
    stats[1] = n_coded;
  }
  return ORC_OK;
}

int orc_decode_rans(const uint8_t* in, uint64_t in_size, uint16_t* y, uint64_t n, uint32_t B, uint8_t* cache) {
  const int ciera = (B != 0);
  if (in == NULL || (n > 0 && y == NULL) || (ciera && n > 0 && cache == NULL)) return ORC_ERR_ARG;
  if (n > ORC_MAX_N || (ciera && !valid_block_size(B))) return ORC_ERR_ARG;
  const uint64_t nchunks = ceil_div(n, ORC_CHUNK);
  const uint64_t sm_pos = rans_sm_pos(nchunks);
  const uint64_t bm_pos = sm_pos + pad128(n);
  const uint64_t pay_pos = bm_pos + (ciera ? 128ull * nchunks : 0);
  if (in_size < pay_pos) return ORC_ERR_FORMAT;
  if (memcmp(in, ciera ? "CIER" : "ZIP3", 4) != 0 || get_u16(in + 4) != ORC_RANS_VERSION ||
      in[6] != (ciera ? 3 : 2) || in[7] != 0 || get_u64(in + 8) != n || get_u32(in + 16) != B ||
      get_u32(in + 20) != ORC_CHUNK || get_u64(in + 24) != nchunks || get_u64(in + 32) > in_size)
    return ORC_ERR_FORMAT;
  const uint64_t total = get_u64(in + 32); /* in_size may exceed it: the rest is not read */
  for (unsigned k = 56; k < ORC_HEADER; k++)
    if (in[k]) return ORC_ERR_FORMAT;
  if (get_u64(in + ORC_HEADER) != pay_pos || get_u64(in + ORC_HEADER + 8 * nchunks) != total)
    return ORC_ERR_FORMAT;
  uint8_t* sym = (uint8_t*)malloc(ORC_CHUNK);
  uint64_t n_changed = 0, n_coded = 0;
  int st = ORC_OK;
  for (uint64_t c = 0; c < nchunks && st == ORC_OK; c++) {
    uint64_t a = get_u64(in + ORC_HEADER + 8 * c), b = get_u64(in + ORC_HEADER + 8 * (c + 1));
    if (b < a || b > total || (a & 127u) || (b & 127u)) {
      st = ORC_ERR_FORMAT;
      break;
    }
    uint64_t m[4], total = 0;
    for (unsigned h = 0; h < 4; h++) {
      uint64_t begin = c * ORC_CHUNK + h * ORC_PART;
      uint64_t end = begin + ORC_PART < n ? begin + ORC_PART : n;
      m[h] = 0;
      for (uint64_t i = begin; i < end; i++) m[h] += (uint64_t)rans_bit(in, bm_pos, B, i);
      total += m[h];
    }
    n_coded += total;
    if (total == 0) {
      if (b != a) st = ORC_ERR_FORMAT;
      continue;
    }
    if (b - a < ORC_RANS_HEAD) {
      st = ORC_ERR_FORMAT;
      break;
    }
    uint64_t words = 0;
    for (unsigned h = 0; h < 4; h++) words += get_u16(in + a + 4 + 2 * h);
    uint64_t len = ORC_RANS_HEAD + 2ull * (in[a + 1] >= in[a] ? in[a + 1] - in[a] + 1u : 0) + 2ull * words;
    if (pad128(len) != b - a) {
      st = ORC_ERR_FORMAT;
      break;
    }
    for (uint64_t k = a + len; k < b; k++)
      if (in[k]) st = ORC_ERR_FORMAT;
    if (st == ORC_OK) st = rans_decode_chunk(in + a, len, m, sym);
    if (st != ORC_OK) break;
    uint64_t k = 0;
    for (uint64_t i = c * ORC_CHUNK; i < n && i < (c + 1) * ORC_CHUNK; i++) {
      if (rans_bit(in, bm_pos, B, i)) {
        y[i] = join_fields(in[sm_pos + i], sym[k++]);
        if (ciera) cache[i] = (uint8_t)exp_field(y[i]);
      }
    }
  }
  free(sym);
  if (st != ORC_OK) return st;
  /* values of unchanged blocks */
  for (uint64_t i = 0; i < n; i++)
    if (!rans_bit(in, bm_pos, B, i)) y[i] = join_fields(in[sm_pos + i], cache[i]);
  if (ciera) {
    for (uint64_t c = 0; c < nchunks; c++) {
      uint64_t nb_c = ceil_div((n - c * ORC_CHUNK < ORC_CHUNK) ? n - c * ORC_CHUNK : ORC_CHUNK, B);
      for (uint64_t j = 0; j < 1024; j++) {
        int bit = (in[bm_pos + 128 * c + (j >> 3)] >> (j & 7)) & 1;
        if (bit && j >= nb_c) return ORC_ERR_FORMAT;
        n_changed += bit;
      }
    }
  }
  if (get_u64(in + 40) != n_changed || get_u64(in + 48) != n_coded) return ORC_ERR_FORMAT;
  return ORC_OK;
}
