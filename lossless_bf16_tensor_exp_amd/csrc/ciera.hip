// ciera.hip -- HIP kernels and C ABI of the lossless BF16 codec, gfx950.
//
// Encode is three kernels on the caller's stream:
//   k_stats  one workgroup per 65,536-value chunk: FP64 partial sums for the
//            tensor's variance (ZipCCL research digest, section 3.1: sigma
//            from one standard-deviation pass) and, in ciera mode, the
//            changed-block bitmap against the sender's exponent cache plus the
//            cache update (CIERA page, section 3.1).
//   k_plan   one workgroup: reduces the partials in a fixed order, picks the
//            window base E0 (integer nearest x_opt = log2 sigma + 0.5 log2(14
//            ln2 / 16383), section 3.1 of the digest, as var >= K0 4^k), and
//            writes the header's size-independent fields.
//   k_write  one workgroup per chunk: splits values into sign+mantissa bytes
//            and 3-bit codes, compacts escapes with wave scans, finds its
//            chunk's stream offset with a decoupled look-back over the
//            preceding chunks' sizes, and writes the 128-byte-aligned
//            sections (digest, section 3.1 last paragraph, and Figure 1).
// Decode is one kernel, k_decode, one workgroup per chunk; chunks are
// independent because the chunk table holds every offset.
//
// Work mapping: a "unit" is 8 consecutive values (one 16-byte load).  A chunk
// has 8192 units; thread t of the 1024-thread workgroup handles units
// j*1024 + t, j = 0..7, so each wave instruction touches 1 KiB of contiguous
// input.  Blocks (B >= 64) never split a unit, and chunks never split a block.
// All data movement is integer: sign, NaN payloads, subnormals and -0 never
// pass through floating-point registers.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include "ciera.h"

namespace {

constexpr uint32_t kChunk = 65536u;
constexpr uint32_t kThreads = 1024u;
constexpr uint32_t kWaves = kThreads / 64u;
constexpr uint32_t kUnitsPerChunk = kChunk / 8u;
constexpr uint32_t kUnitsPerThread = kUnitsPerChunk / kThreads;  // 8
constexpr uint32_t kBitmapWords = 32u;  // 1024 blocks per chunk at B = 64
constexpr uint64_t kMaxN = 1ull << 40;
constexpr uint64_t kHeader = 128u;
constexpr uint32_t kMaxE0 = 249u;
// 16383 / (28 ln 2) as a double: the variance threshold of window base k is
// kK0 * 4^k.
constexpr double kK0 = 0x1.a610ca4a234eep+9;
// Look-back status words: two flag bits over a 62-bit byte count.
constexpr uint64_t kFlagAggregate = 1ull << 62;
constexpr uint64_t kFlagInclusive = 2ull << 62;
constexpr uint64_t kValueMask = (1ull << 62) - 1u;
constexpr uint32_t kSpinLimit = 1u << 26;

__host__ __device__ inline uint64_t pad128(uint64_t v) { return (v + 127u) & ~uint64_t(127); }
__host__ __device__ inline uint64_t cdiv(uint64_t a, uint64_t b) { return (a + b - 1u) / b; }
__host__ __device__ inline uint64_t table_end(uint64_t nchunks) {
  return kHeader + pad128(8u * (nchunks + 1u));
}

// Workspace: a control block, one error word per chunk, per-chunk partial
// sums, per-chunk bitmap words (ciera) and per-chunk look-back words.
struct Ctrl {
  uint32_t e0;
  uint32_t ticket;
  uint64_t esc_total;
  uint64_t n_err_slots;
  uint64_t reserved[29];
};
static_assert(sizeof(Ctrl) == 256, "control block is 256 bytes");

struct Partial {
  double s1;
  double s2;
  uint32_t nf;
  uint32_t nch;
  uint32_t pad[2];
};

struct WsLayout {
  uint64_t err, partial, bitmap, status, total;
};

__host__ __device__ inline uint64_t align256(uint64_t v) { return (v + 255u) & ~uint64_t(255); }

__host__ inline WsLayout ws_layout(uint64_t nchunks) {
  WsLayout l;
  const uint64_t slots = nchunks ? nchunks : 1u;
  l.err = sizeof(Ctrl);
  l.partial = align256(l.err + 4u * slots);
  l.bitmap = align256(l.partial + sizeof(Partial) * slots);
  l.status = align256(l.bitmap + 4u * kBitmapWords * slots);
  l.total = align256(l.status + 8u * slots);
  return l;
}

struct Ws {
  Ctrl* ctrl;
  uint32_t* err;
  Partial* partial;
  uint32_t* bitmap;
  uint64_t* status;
};

__host__ inline Ws ws_bind(void* base, uint64_t nchunks) {
  const WsLayout l = ws_layout(nchunks);
  uint8_t* b = static_cast<uint8_t*>(base);
  Ws w;
  w.ctrl = reinterpret_cast<Ctrl*>(b);
  w.err = reinterpret_cast<uint32_t*>(b + l.err);
  w.partial = reinterpret_cast<Partial*>(b + l.partial);
  w.bitmap = reinterpret_cast<uint32_t*>(b + l.bitmap);
  w.status = reinterpret_cast<uint64_t*>(b + l.status);
  return w;
}

// ------------------------------------------------------------------ device helpers
__device__ inline uint32_t lane_id() { return threadIdx.x & 63u; }

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// v_perm_b32: byte i of the result is byte sel_i of {b (0..3), a (4..7)};
// selector 0x0C yields a zero byte.
__device__ inline uint32_t perm(uint32_t a, uint32_t b, uint32_t sel) { return __builtin_amdgcn_perm(a, b, sel); }
// bits of a where mask is set, bits of b elsewhere (v_bfi_b32)
__device__ inline uint32_t bfi(uint32_t mask, uint32_t a, uint32_t b) { return (mask & a) | (~mask & b); }

// Eight BF16 patterns (a "unit"): w[i] holds value 2i in its low and value
// 2i+1 in its high half.  Values past the data read as zero.
struct Unit {
  uint32_t w[4];
};

__device__ inline Unit load_unit(const uint16_t* __restrict__ x, uint64_t first, uint32_t cnt) {
  Unit u;
  if (cnt == 8u) {
    const uint4 v = *reinterpret_cast<const uint4*>(x + first);
    u.w[0] = v.x;
    u.w[1] = v.y;
    u.w[2] = v.z;
    u.w[3] = v.w;
  } else {
    for (int i = 0; i < 4; i++) u.w[i] = 0u;
    for (uint32_t k = 0; k < cnt; k++) u.w[k >> 1] |= uint32_t(x[first + k]) << (16u * (k & 1u));
  }
  return u;
}

__device__ inline void store_unit(uint16_t* __restrict__ y, uint64_t first, uint32_t cnt, const Unit& u) {
  if (cnt == 8u) {
    *reinterpret_cast<uint4*>(y + first) = make_uint4(u.w[0], u.w[1], u.w[2], u.w[3]);
  } else {
    for (uint32_t k = 0; k < cnt; k++) y[first + k] = uint16_t(u.w[k >> 1] >> (16u * (k & 1u)));
  }
}

__device__ inline uint2 load_bytes8(const uint8_t* __restrict__ p, uint32_t cnt) {
  if (cnt == 8u) return *reinterpret_cast<const uint2*>(p);
  uint2 v = make_uint2(0u, 0u);
  for (uint32_t k = 0; k < cnt; k++) {
    if (k < 4u)
      v.x |= uint32_t(p[k]) << (8u * k);
    else
      v.y |= uint32_t(p[k]) << (8u * (k - 4u));
  }
  return v;
}

__device__ inline void store_bytes8(uint8_t* __restrict__ p, uint32_t cnt, uint2 v) {
  if (cnt == 8u) {
    *reinterpret_cast<uint2*>(p) = v;
  } else {
    for (uint32_t k = 0; k < cnt; k++) p[k] = uint8_t((k < 4u ? v.x : v.y) >> (8u * (k & 3u)));
  }
}

// Exponent fields as 16-bit lanes: bits 0..7 = exponent of the low value,
// bits 16..23 = exponent of the high value.
__device__ inline uint32_t exp_pair(uint32_t w) { return (w >> 7) & 0x00FF00FFu; }

// Exponent bytes of the unit: byte k of {lo, hi} = exponent of value k.
__device__ inline uint2 unit_exponents(const Unit& u) {
  return make_uint2(perm(exp_pair(u.w[1]), exp_pair(u.w[0]), 0x06040200u),
                    perm(exp_pair(u.w[3]), exp_pair(u.w[2]), 0x06040200u));
}

// Sign+mantissa bytes: byte k = (sign << 7) | mantissa of value k.
__device__ inline uint2 unit_sm(const Unit& u) {
  uint32_t s[4];
#pragma unroll
  for (int i = 0; i < 4; i++) s[i] = bfi(0x00800080u, u.w[i] >> 8, u.w[i]);
  return make_uint2(perm(s[1], s[0], 0x06040200u), perm(s[3], s[2], 0x06040200u));
}

// 3-bit codes of an exponent pair as 16-bit lanes: min(E - E0 + 1, 8) with
// 16-bit wrap-around, i.e. 1..7 inside the window, 0 or 8 outside.  Bits
// 0..2 of each lane are the code (8 has code bits 000).
__device__ inline uint32_t code_pair(uint32_t e, uint32_t bias /* (1 - E0) in both lanes */) {
  const u16x2 s = __builtin_bit_cast(u16x2, e) + __builtin_bit_cast(u16x2, bias);
  const u16x2 eight = {8, 8};
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_min(s, eight));
}

// The three code planes of a unit, byte b = plane b (bit k = bit b of the
// code of value k), from the four code pairs.
__device__ inline uint32_t unit_planes(const uint32_t (&c)[4]) {
  // nibble i = code of value 2i, nibble 4+i = code of value 2i+1
  const uint32_t q = c[0] | (c[1] << 4) | (c[2] << 8) | (c[3] << 12);
  uint32_t planes = 0;
#pragma unroll
  for (uint32_t b = 0; b < 3u; b++) {
    uint32_t t = (q >> b) & 0x11111111u;  // even values at 4i, odd values at 16+4i
    t = (t | (t >> 15)) & 0x3333u;       // (even, odd) pairs at 4i, 4i+1
    t = (t | (t >> 2)) & 0x0F0Fu;
    t = (t | (t >> 4)) & 0x00FFu;
    planes |= t << (8u * b);
  }
  return planes;
}

// Inverse of unit_planes for one half: bits k (k < 4) of the 4-bit value x
// spread to bit 0 of byte k (the multiply's cross terms never land on a
// multiple of 8).
__device__ inline uint32_t spread4(uint32_t x) { return (x * 0x00204081u) & 0x01010101u; }

// Code bytes (0..7) of a unit from its three plane bytes: lo = values 0..3,
// hi = values 4..7.
__device__ inline uint2 codes_from_planes(uint32_t p0, uint32_t p1, uint32_t p2) {
  const uint32_t lo = spread4(p0 & 15u) | (spread4(p1 & 15u) << 1) | (spread4(p2 & 15u) << 2);
  const uint32_t hi = spread4(p0 >> 4) | (spread4(p1 >> 4) << 1) | (spread4(p2 >> 4) << 2);
  return make_uint2(lo, hi);
}

// Exponent bytes E0 + code - 1 for code bytes 1..7; code-0 bytes give junk
// that the escape pass replaces.  No carry or borrow crosses a byte: with
// E0 >= 1 every byte sum is at most 7 + 248; with E0 = 0 each byte is first
// lifted by 0x80 so the subtraction cannot borrow.
__device__ inline uint32_t exps_from_codes(uint32_t codes, uint32_t e0) {
  return e0 ? codes + (e0 - 1u) * 0x01010101u : ((codes | 0x80808080u) - 0x01010101u) & 0x7F7F7F7Fu;
}

// Two output values from byte pairs: h = sm_a | E_a << 8 | sm_b << 16 | E_b << 24.
__device__ inline uint32_t join_pair(uint32_t h) {
  // bits 0..6 mantissa from sm, 7..14 exponent, 15 sign (sm bit 7)
  return bfi(0x007F007Fu, h, bfi(0x80008000u, h << 8, h >> 1));
}

__device__ inline Unit unit_join(uint2 sm, uint2 e) {
  Unit o;
  o.w[0] = join_pair(perm(e.x, sm.x, 0x05010400u));
  o.w[1] = join_pair(perm(e.x, sm.x, 0x07030602u));
  o.w[2] = join_pair(perm(e.y, sm.y, 0x05010400u));
  o.w[3] = join_pair(perm(e.y, sm.y, 0x07030602u));
  return o;
}

__device__ inline uint32_t byte_of(uint2 v, uint32_t k) { return ((k < 4u ? v.x : v.y) >> (8u * (k & 3u))) & 0xFFu; }

__device__ inline uint2 set_byte(uint2 v, uint32_t k, uint32_t b) {
  const uint32_t sh = 8u * (k & 3u);
  const uint32_t m = ~(0xFFu << sh);
  if (k < 4u)
    v.x = (v.x & m) | (b << sh);
  else
    v.y = (v.y & m) | (b << sh);
  return v;
}

__device__ inline uint32_t wave_incl_scan(uint32_t v) {
  const uint32_t lane = lane_id();
#pragma unroll
  for (uint32_t d = 1; d < 64u; d <<= 1) {
    const uint32_t t = __shfl_up(v, d, 64);
    if (lane >= d) v += t;
  }
  return v;
}

__device__ inline double wave_sum(double v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
  return v;
}

__device__ inline uint64_t wave_sum_u64(uint64_t v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
  return v;
}

__device__ inline uint32_t wave_sum_u32(uint32_t v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
  return v;
}

// Escape positions: each thread holds kUnitsPerThread counts (one per unit,
// 0..8), units ordered (j, wave, lane).  On return base[j] is the number of
// escapes in all earlier units of the chunk and the function returns the
// chunk total.  Every thread of the workgroup must call it.
__device__ inline uint32_t chunk_escape_scan(const uint32_t (&cnt)[kUnitsPerThread],
                                             uint32_t (&base)[kUnitsPerThread],
                                             uint32_t* s_tot /* kUnitsPerThread*kWaves + 1 */) {
  const uint32_t lane = lane_id();
  const uint32_t wave = threadIdx.x >> 6;
  // two counts per 32-bit word (16-bit fields; a wave's sum is at most 512)
#pragma unroll
  for (uint32_t p = 0; p < kUnitsPerThread / 2u; p++) {
    const uint32_t packed = cnt[2 * p] | (cnt[2 * p + 1] << 16);
    const uint32_t incl = wave_incl_scan(packed);
    const uint32_t excl = incl - packed;
    base[2 * p] = excl & 0xFFFFu;
    base[2 * p + 1] = excl >> 16;
    if (lane == 63u) {
      s_tot[(2 * p) * kWaves + wave] = incl & 0xFFFFu;
      s_tot[(2 * p + 1) * kWaves + wave] = incl >> 16;
    }
  }
  __syncthreads();
  // exclusive scan of the kUnitsPerThread*kWaves totals in (j, wave) order,
  // by wave 0: lane l owns entries 2l and 2l+1
  if (wave == 0) {
    const uint32_t a = s_tot[2 * lane], b = s_tot[2 * lane + 1];
    const uint32_t incl = wave_incl_scan(a + b);
    const uint32_t excl = incl - (a + b);
    s_tot[2 * lane] = excl;
    s_tot[2 * lane + 1] = excl + a;
    if (lane == 63u) s_tot[kUnitsPerThread * kWaves] = incl;
  }
  __syncthreads();
#pragma unroll
  for (uint32_t j = 0; j < kUnitsPerThread; j++) base[j] += s_tot[j * kWaves + wave];
  return s_tot[kUnitsPerThread * kWaves];
}

// ------------------------------------------------------------------ k_stats
// FP64 value of a BF16 pattern held in the top half of a float: BF16 -> FP32
// is exact (denormals are kept), FP32 -> FP64 is exact.
__device__ inline double widen_hi(uint32_t hi_bits) { return double(__uint_as_float(hi_bits)); }

// Partial sums of one unit's finite values (the checked path).
__device__ inline void stats_checked(const Unit& v, uint32_t cnt, double shift, double& s1, double& s2,
                                     uint32_t& nf) {
  for (uint32_t k = 0; k < cnt; k++) {
    const uint32_t b = (v.w[k >> 1] >> (16u * (k & 1u))) & 0xFFFFu;
    if (((b >> 7) & 0xFFu) == 0xFFu) continue;
    const double d = widen_hi(b << 16) - shift;
    s1 += d;
    s2 = fma(d, d, s2);
    nf++;
  }
}

template <bool kCiera>
__global__ __launch_bounds__(kThreads) void k_stats(const uint16_t* __restrict__ x, uint64_t n,
                                                    uint8_t* __restrict__ cache, uint32_t log2B, Ws ws) {
  __shared__ uint32_t s_bits[kBitmapWords];
  __shared__ double s_s1[kWaves], s_s2[kWaves];
  __shared__ uint32_t s_nf[kWaves];
  const uint32_t tid = threadIdx.x;
  const uint32_t c = blockIdx.x;
  const uint64_t start = uint64_t(c) * kChunk;
  const uint32_t nc = uint32_t(min(uint64_t(kChunk), n - start));
  const uint32_t nunits = (nc + 7u) / 8u;
  if (kCiera && tid < kBitmapWords) s_bits[tid] = 0u;
  const uint32_t first = x[0];
  const double shift = (((first >> 7) & 0xFFu) != 0xFFu) ? widen_hi(first << 16) : 0.0;
  __syncthreads();

  // Fast path: no finite test per value.  A non-finite input makes the
  // thread's sums non-finite (squares of finite BF16 values cannot
  // overflow FP64), and the thread then redoes its units on the checked path.
  double s1 = 0.0, s2 = 0.0;
  uint32_t nf = 0;
#pragma unroll
  for (uint32_t j = 0; j < kUnitsPerThread; j++) {
    const uint32_t u = j * kThreads + tid;
    if (u < nunits) {
      const uint32_t cnt = min(8u, nc - 8u * u);
      const uint64_t at = start + 8ull * u;
      const Unit v = load_unit(x, at, cnt);
      if (cnt == 8u) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const double lo = widen_hi(v.w[i] << 16) - shift;
          const double hi = widen_hi(v.w[i] & 0xFFFF0000u) - shift;
          s1 += lo;
          s2 = fma(lo, lo, s2);
          s1 += hi;
          s2 = fma(hi, hi, s2);
        }
        nf += 8u;
      } else {
        stats_checked(v, cnt, shift, s1, s2, nf);
      }
      if (kCiera) {
        const uint2 e = unit_exponents(v);
        const uint2 old = load_bytes8(cache + at, cnt);
        const uint64_t keep = (cnt == 8u) ? ~0ull : ((1ull << (8u * cnt)) - 1u);
        const uint64_t diff = ((uint64_t(e.y ^ old.y) << 32) | (e.x ^ old.x)) & keep;
        if (diff) {
          store_bytes8(cache + at, cnt, e);
          const uint32_t blk = (8u * u) >> log2B;
          atomicOr(&s_bits[blk >> 5], 1u << (blk & 31u));
        }
      }
    }
  }
  if (!(__builtin_isfinite(s1) && __builtin_isfinite(s2))) {
    s1 = 0.0;
    s2 = 0.0;
    nf = 0;
    for (uint32_t j = 0; j < kUnitsPerThread; j++) {
      const uint32_t u = j * kThreads + tid;
      if (u >= nunits) break;
      const uint32_t cnt = min(8u, nc - 8u * u);
      stats_checked(load_unit(x, start + 8ull * u, cnt), cnt, shift, s1, s2, nf);
    }
  }
  s1 = wave_sum(s1);
  s2 = wave_sum(s2);
  nf = wave_sum_u32(nf);
  if (lane_id() == 0u) {
    s_s1[tid >> 6] = s1;
    s_s2[tid >> 6] = s2;
    s_nf[tid >> 6] = nf;
  }
  __syncthreads();
  if (tid == 0) {
    double a = 0.0, b = 0.0;
    uint32_t m = 0;
    for (uint32_t w = 0; w < kWaves; w++) {
      a += s_s1[w];
      b += s_s2[w];
      m += s_nf[w];
    }
    uint32_t nch = 0;
    if (kCiera)
      for (uint32_t w = 0; w < kBitmapWords; w++) nch += __popc(s_bits[w]);
    Partial p;
    p.s1 = a;
    p.s2 = b;
    p.nf = m;
    p.nch = nch;
    p.pad[0] = p.pad[1] = 0u;
    ws.partial[c] = p;
    ws.status[c] = 0u;
  }
  if (kCiera && tid < kBitmapWords) ws.bitmap[uint64_t(c) * kBitmapWords + tid] = s_bits[tid];
}

// ------------------------------------------------------------------ k_plan
// Window base: E0 = 127 + k for the largest k with var >= K0 * 4^k, clamped
// to [0, 249]; 0 without a finite spread.  The comparisons are exact: each
// threshold is a power of two times K0.
__device__ inline uint32_t window_base(double var, uint64_t nf) {
  if (nf < 2u || !(var > 0.0)) return 0u;
  // K0 lies in [2^9, 2^10), so var >= K0 * 4^k holds for k = floor((t-11)/2)
  // with t = ilogb(var), and fails for k > (t-8)/2: start low, step up.
  const int t = ilogb(var);
  int k = (t - 11 >= 0) ? (t - 11) / 2 : -((12 - t) / 2);
  if (k < -128) k = -128;
  if (k > 122) k = 122;  // var >= K0 * 4^122 already
  while (k < 122 && var >= ldexp(kK0, 2 * (k + 1))) k++;
  return k < -127 ? 0u : uint32_t(127 + k);
}

__global__ __launch_bounds__(kThreads) void k_plan(uint64_t n, uint64_t nchunks, uint32_t B, int e0_override,
                                                   uint8_t* __restrict__ out, uint64_t* __restrict__ out_size,
                                                   Ws ws) {
  __shared__ double s_s1[kWaves], s_s2[kWaves];
  __shared__ uint64_t s_nf[kWaves], s_nch[kWaves];
  const uint32_t tid = threadIdx.x;
  double a = 0.0, b = 0.0;
  uint64_t m = 0, q = 0;
  for (uint64_t c = tid; c < nchunks; c += kThreads) {
    const Partial p = ws.partial[c];
    a += p.s1;
    b += p.s2;
    m += p.nf;
    q += p.nch;
  }
  a = wave_sum(a);
  b = wave_sum(b);
  m = wave_sum_u64(m);
  q = wave_sum_u64(q);
  if (lane_id() == 0u) {
    s_s1[tid >> 6] = a;
    s_s2[tid >> 6] = b;
    s_nf[tid >> 6] = m;
    s_nch[tid >> 6] = q;
  }
  uint64_t* table = reinterpret_cast<uint64_t*>(out + kHeader);
  const uint64_t base = table_end(nchunks);
  // zero the table's padding words (entries past nchunks)
  for (uint64_t i = nchunks + 1u + tid; i < (base - kHeader) / 8u; i += kThreads) table[i] = 0u;
  __syncthreads();
  if (tid == 0) {
    double s1 = 0.0, s2 = 0.0;
    uint64_t nf = 0, nch = 0;
    for (uint32_t w = 0; w < kWaves; w++) {
      s1 += s_s1[w];
      s2 += s_s2[w];
      nf += s_nf[w];
      nch += s_nch[w];
    }
    double var = 0.0;
    if (nf >= 2u) {
      var = (s2 - s1 * s1 / double(nf)) / double(nf - 1u);
      if (!(var > 0.0)) var = 0.0;
    }
    const uint32_t e0 = (e0_override >= 0) ? uint32_t(e0_override) : window_base(var, nf);
    ws.ctrl->e0 = e0;
    ws.ctrl->ticket = 0u;
    ws.ctrl->esc_total = 0u;
    ws.ctrl->n_err_slots = nchunks;
    const uint32_t magic = B ? 0x52454943u /* "CIER" */ : 0x3350495Au /* "ZIP3" */;
    uint64_t* h = reinterpret_cast<uint64_t*>(out);
    h[0] = uint64_t(magic) | (1ull << 32) | (uint64_t(B ? 1u : 0u) << 48) | (uint64_t(e0) << 56);
    h[1] = n;
    h[2] = uint64_t(B) | (uint64_t(kChunk) << 32);
    h[3] = nchunks;
    h[5] = nch;
    for (int i = 7; i < 16; i++) h[i] = 0u;
    if (nchunks == 0u) {
      h[4] = base;
      h[6] = 0u;
      table[0] = base;
      *out_size = base;
    }
  }
}

// ------------------------------------------------------------------ k_write
// Per-chunk static geometry shared by encode and decode.
struct ChunkGeom {
  uint64_t sm, bitmap, plane, esc;  // absolute section offsets
  uint64_t plane_bytes;             // padded size of one plane
};

__device__ inline ChunkGeom chunk_geom(uint64_t begin, uint32_t nc, bool ciera, uint32_t nch, uint32_t B) {
  ChunkGeom g;
  g.sm = begin;
  g.bitmap = g.sm + pad128(nc);
  const uint64_t after_bitmap = g.bitmap + (ciera ? 128u : 0u);
  const uint64_t p = ciera ? uint64_t(nch) * B / 8u : cdiv(nc, 8u);
  g.plane_bytes = pad128(p);
  g.plane = after_bitmap;
  g.esc = g.plane + 3u * g.plane_bytes;
  return g;
}

__device__ inline void zero_fill(uint8_t* __restrict__ p, uint64_t from, uint64_t to) {
  for (uint64_t i = from + threadIdx.x; i < to; i += kThreads) p[i] = 0u;
}

// Decoupled look-back, run by one whole wave: publish this chunk's size as an
// aggregate, then sum predecessors' published sizes 64 at a time until one
// holds an inclusive prefix; publish the inclusive prefix.  Predecessors
// always hold earlier tickets, so their workgroups are already running and
// publish their aggregates without waiting on anything.  Returns the byte
// offset of this chunk relative to the first chunk; sets *err if a wait
// exceeds kSpinLimit polls.
__device__ inline uint64_t look_back(uint64_t* __restrict__ status, uint32_t c, uint64_t size, uint32_t* err) {
  const uint32_t lane = lane_id();
  if (c == 0u) {
    if (lane == 0u)
      __hip_atomic_store(&status[0], kFlagInclusive | size, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    return 0u;
  }
  if (lane == 0u)
    __hip_atomic_store(&status[c], kFlagAggregate | size, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
  uint64_t prefix = 0;
  int64_t top = int64_t(c) - 1;  // closest predecessor not yet summed
  uint32_t spins = 0;
  while (true) {
    const int64_t k = top - int64_t(lane);
    const uint64_t s = (k >= 0) ? __hip_atomic_load(&status[k], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT)
                                : kFlagInclusive;  // before chunk 0: an empty inclusive prefix
    const uint64_t flag = s & ~kValueMask;
    if (__ballot(flag == 0u) != 0u) {
      if (++spins > kSpinLimit) {
        *err = CIERA_ERR_INTERNAL;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
      continue;
    }
    const uint64_t incl = __ballot(flag == kFlagInclusive);
    if (incl != 0u) {
      const uint32_t first = uint32_t(__builtin_ctzll(incl));  // closest inclusive predecessor
      prefix += wave_sum_u64(lane <= first ? (s & kValueMask) : 0u);
      break;
    }
    prefix += wave_sum_u64(s & kValueMask);
    top -= 64;
  }
  if (lane == 0u)
    __hip_atomic_store(&status[c], kFlagInclusive | (prefix + size), __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
  return prefix;
}

template <bool kCiera>
__global__ __launch_bounds__(kThreads) void k_write(const uint16_t* __restrict__ x, uint64_t n, uint64_t nchunks,
                                                    uint32_t log2B, uint8_t* __restrict__ out,
                                                    uint64_t* __restrict__ out_size, Ws ws) {
  __shared__ uint32_t s_chunk;
  __shared__ uint32_t s_bits[kBitmapWords];
  __shared__ uint32_t s_rank[kBitmapWords];
  __shared__ uint32_t s_tot[kUnitsPerThread * kWaves + 1];
  __shared__ uint64_t s_begin;
  __shared__ uint32_t s_err;
  const uint32_t tid = threadIdx.x;
  const uint32_t B = 1u << log2B;
  if (tid == 0) s_chunk = atomicAdd(&ws.ctrl->ticket, 1u);
  __syncthreads();
  const uint32_t c = s_chunk;
  const uint64_t start = uint64_t(c) * kChunk;
  const uint32_t nc = uint32_t(min(uint64_t(kChunk), n - start));
  const uint32_t nunits = (nc + 7u) / 8u;
  const uint32_t e0 = ws.ctrl->e0;
  const uint32_t bias = ((1u - e0) & 0xFFFFu) * 0x00010001u;

  uint32_t nch = 0;
  if (kCiera) {
    if (tid < 64u) {
      const uint32_t w = (tid < kBitmapWords) ? ws.bitmap[uint64_t(c) * kBitmapWords + tid] : 0u;
      const uint32_t pc = __popc(w);
      const uint32_t incl = wave_incl_scan(pc);
      if (tid < kBitmapWords) {
        s_bits[tid] = w;
        s_rank[tid] = incl - pc;
      }
    }
    __syncthreads();
    nch = s_rank[kBitmapWords - 1] + __popc(s_bits[kBitmapWords - 1]);
  }

  // Load the chunk; per unit: the three plane bytes and the escape mask.
  Unit v[kUnitsPerThread];
  uint32_t cnt[kUnitsPerThread], base[kUnitsPerThread];
  uint32_t planes[kUnitsPerThread];  // p0 | p1 << 8 | p2 << 16 | escape mask << 24
#pragma unroll
  for (uint32_t j = 0; j < kUnitsPerThread; j++) {
    const uint32_t u = j * kThreads + tid;
    cnt[j] = 0u;
    planes[j] = 0u;
    v[j].w[0] = v[j].w[1] = v[j].w[2] = v[j].w[3] = 0u;
    if (u < nunits) {
      const uint32_t valid = min(8u, nc - 8u * u);
      v[j] = load_unit(x, start + 8ull * u, valid);
    }
  }
#pragma unroll
  for (uint32_t j = 0; j < kUnitsPerThread; j++) {
    const uint32_t u = j * kThreads + tid;
    if (u < nunits) {
      bool coded = true;
      if (kCiera) {
        const uint32_t blk = (8u * u) >> log2B;
        coded = (s_bits[blk >> 5] >> (blk & 31u)) & 1u;
      }
      if (coded) {
        const uint32_t valid = min(8u, nc - 8u * u);
        const uint32_t vmask = (valid == 8u) ? 0xFFu : ((1u << valid) - 1u);
        uint32_t cp[4];
#pragma unroll
        for (int i = 0; i < 4; i++) cp[i] = code_pair(exp_pair(v[j].w[i]), bias);
        uint32_t p = unit_planes(cp) & (vmask * 0x010101u);
        const uint32_t em = ~(p | (p >> 8) | (p >> 16)) & vmask;
        planes[j] = p | (em << 24);
        cnt[j] = __popc(em);
      }
    }
  }
  const uint32_t nesc = chunk_escape_scan(cnt, base, s_tot);

  // Chunk size, then its offset by look-back over earlier chunks (wave 0).
  const uint64_t size = pad128(nc) + (kCiera ? 128u : 0u) +
                        3u * pad128(kCiera ? uint64_t(nch) * B / 8u : cdiv(nc, 8u)) + pad128(nesc);
  if (tid < 64u) {
    if (tid == 0)
      atomicAdd(reinterpret_cast<unsigned long long*>(&ws.ctrl->esc_total), (unsigned long long)nesc);
    uint32_t err = 0u;
    const uint64_t prefix = look_back(ws.status, c, size, &err);
    if (tid == 0) {
      const uint64_t begin = table_end(nchunks) + prefix;
      s_begin = begin;
      s_err = err;
      ws.err[c] = err;
      uint64_t* table = reinterpret_cast<uint64_t*>(out + kHeader);
      table[c] = begin;
      if (uint64_t(c) + 1u == nchunks) {
        const uint64_t total = begin + size;
        table[nchunks] = total;
        uint64_t* h = reinterpret_cast<uint64_t*>(out);
        h[4] = total;
        h[6] = __hip_atomic_load(&ws.ctrl->esc_total, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
        *out_size = total;
      }
    }
  }
  __syncthreads();
  if (s_err) return;  // uniform; the error word tells the caller
  const ChunkGeom g = chunk_geom(s_begin, nc, kCiera, nch, B);

  // Write sections.
#pragma unroll
  for (uint32_t j = 0; j < kUnitsPerThread; j++) {
    const uint32_t u = j * kThreads + tid;
    if (u >= nunits) continue;
    *reinterpret_cast<uint2*>(out + g.sm + 8ull * u) = unit_sm(v[j]);
    bool coded = true;
    uint64_t pbyte = u;
    if (kCiera) {
      const uint32_t blk = (8u * u) >> log2B;
      const uint32_t word = s_bits[blk >> 5];
      coded = (word >> (blk & 31u)) & 1u;
      const uint32_t rank = s_rank[blk >> 5] + __popc(word & ((1u << (blk & 31u)) - 1u));
      pbyte = uint64_t(rank) * (B / 8u) + (u & (B / 8u - 1u));
    }
    if (coded) {
      const uint32_t p = planes[j];
      out[g.plane + pbyte] = uint8_t(p);
      out[g.plane + g.plane_bytes + pbyte] = uint8_t(p >> 8);
      out[g.plane + 2u * g.plane_bytes + pbyte] = uint8_t(p >> 16);
      uint32_t em = p >> 24;
      if (em) {
        const uint2 e = unit_exponents(v[j]);
        uint64_t at = g.esc + base[j];
        while (em) {
          const uint32_t k = __builtin_ctz(em);
          em &= em - 1u;
          out[at++] = uint8_t(byte_of(e, k));
        }
      }
    }
  }
  if (kCiera && tid < kBitmapWords) *reinterpret_cast<uint32_t*>(out + g.bitmap + 4u * tid) = s_bits[tid];
  // Zero padding after each section's data.
  zero_fill(out, g.sm + 8ull * nunits, g.bitmap);
  uint64_t plane_data;
  if (!kCiera) {
    plane_data = nunits;
  } else {
    const uint32_t last = (nc - 1u) >> log2B;  // last block of the chunk
    const bool last_changed = (s_bits[last >> 5] >> (last & 31u)) & 1u;
    const uint32_t last_rank = s_rank[last >> 5] + __popc(s_bits[last >> 5] & ((1u << (last & 31u)) - 1u));
    plane_data = last_changed ? uint64_t(last_rank) * (B / 8u) + (nunits - last * (B / 8u))
                              : uint64_t(nch) * (B / 8u);
  }
  for (uint32_t b = 0; b < 3u; b++)
    zero_fill(out, g.plane + b * g.plane_bytes + plane_data, g.plane + (b + 1u) * g.plane_bytes);
  zero_fill(out, g.esc + nesc, g.esc + pad128(nesc));
}

// ------------------------------------------------------------------ k_decode
template <bool kCiera>
__global__ __launch_bounds__(kThreads) void k_decode(const uint8_t* __restrict__ in, uint64_t in_size,
                                                     uint16_t* __restrict__ y, uint64_t n, uint64_t nchunks,
                                                     uint32_t log2B, uint8_t* __restrict__ cache,
                                                     uint64_t* __restrict__ n_err_slots,
                                                     uint32_t* __restrict__ err_slots) {
  __shared__ uint32_t s_ok;    // header and table entries are consistent
  __shared__ uint32_t s_fits;  // the chunk's fixed-size sections lie inside it
  __shared__ uint32_t s_e0;
  __shared__ uint64_t s_begin, s_end;
  __shared__ uint32_t s_bits[kBitmapWords];
  __shared__ uint32_t s_rank[kBitmapWords];
  __shared__ uint32_t s_tot[kUnitsPerThread * kWaves + 1];
  const uint32_t tid = threadIdx.x;
  const uint32_t c = blockIdx.x;
  const uint32_t B = kCiera ? (1u << log2B) : 0u;
  const uint64_t base_off = table_end(nchunks);
  if (tid == 0) {
    uint32_t ok = 1u;
    const uint64_t* h = reinterpret_cast<const uint64_t*>(in);
    const uint32_t magic = kCiera ? 0x52454943u : 0x3350495Au;
    uint64_t begin = 0, end = 0;
    uint32_t e0 = 0;
    if (in_size < base_off) {
      ok = 0u;
    } else {
      const uint64_t h0 = h[0];
      e0 = uint32_t(h0 >> 56);
      ok &= uint32_t(h0 & 0xFFFFFFFFu) == magic;
      ok &= ((h0 >> 32) & 0xFFFFu) == 1u;
      ok &= ((h0 >> 48) & 0xFFu) == (kCiera ? 1u : 0u);
      ok &= e0 <= kMaxE0;
      ok &= h[1] == n;
      ok &= h[2] == (uint64_t(B) | (uint64_t(kChunk) << 32));
      ok &= h[3] == nchunks;
      const uint64_t total = h[4];
      ok &= total <= in_size;
      for (int i = 7; i < 16; i++) ok &= h[i] == 0u;
      const uint64_t* table = reinterpret_cast<const uint64_t*>(in + kHeader);
      ok &= table[0] == base_off;
      ok &= table[nchunks] == total;
      if (ok && nchunks) {
        begin = table[c];
        end = table[c + 1u];
        ok &= begin >= base_off && begin <= end && end <= total;
        ok &= ((begin | end) & 127u) == 0u;
      }
    }
    s_ok = ok;
    s_e0 = e0;
    s_begin = begin;
    s_end = end;
    if (c == 0u) *n_err_slots = gridDim.x;
  }
  __syncthreads();
  if (!s_ok || nchunks == 0u) {
    if (tid == 0) err_slots[c] = s_ok ? 0u : uint32_t(CIERA_ERR_FORMAT);
    return;
  }
  const uint32_t e0 = s_e0;
  const uint64_t begin = s_begin, end = s_end;
  const uint64_t start = uint64_t(c) * kChunk;
  const uint32_t nc = uint32_t(min(uint64_t(kChunk), n - start));
  const uint32_t nunits = (nc + 7u) / 8u;

  uint32_t nch = 0;
  if (kCiera) {
    // the bitmap section must lie inside the chunk before it is read
    const uint64_t bm = begin + pad128(nc);
    const bool fits = bm + 128u <= end;
    if (tid < 64u) {
      const uint32_t nb = (nc + B - 1u) >> log2B;
      uint32_t w = 0;
      if (fits && tid < kBitmapWords) {
        w = *reinterpret_cast<const uint32_t*>(in + bm + 4u * tid);
        const uint32_t lo = 32u * tid;
        w = (lo >= nb) ? 0u : (nb - lo >= 32u ? w : (w & ((1u << (nb - lo)) - 1u)));
      }
      const uint32_t pc = __popc(w);
      const uint32_t incl = wave_incl_scan(pc);
      if (tid < kBitmapWords) {
        s_bits[tid] = w;
        s_rank[tid] = incl - pc;
      }
    }
    if (tid == 0) s_fits = fits ? 1u : 0u;
    __syncthreads();
    nch = s_rank[kBitmapWords - 1] + __popc(s_bits[kBitmapWords - 1]);
  } else if (tid == 0) {
    s_fits = 1u;
  }
  __syncthreads();
  const uint32_t bitmap_fits = s_fits;
  const ChunkGeom g = chunk_geom(begin, nc, kCiera, nch, B);
  if (!bitmap_fits || g.esc > end) {
    if (tid == 0) err_slots[c] = uint32_t(CIERA_ERR_FORMAT);
    return;
  }

  uint2 smv[kUnitsPerThread], ev[kUnitsPerThread];
  uint32_t cnt[kUnitsPerThread], base[kUnitsPerThread], emask[kUnitsPerThread];
#pragma unroll
  for (uint32_t j = 0; j < kUnitsPerThread; j++) {
    const uint32_t u = j * kThreads + tid;
    cnt[j] = 0u;
    emask[j] = 0u;
    smv[j] = make_uint2(0u, 0u);
    ev[j] = make_uint2(0u, 0u);
    if (u >= nunits) continue;
    const uint32_t valid = min(8u, nc - 8u * u);
    smv[j] = load_bytes8(in + g.sm + 8ull * u, valid);
    bool coded = true;
    uint64_t pbyte = u;
    if (kCiera) {
      const uint32_t blk = (8u * u) >> log2B;
      const uint32_t word = s_bits[blk >> 5];
      coded = (word >> (blk & 31u)) & 1u;
      const uint32_t rank = s_rank[blk >> 5] + __popc(word & ((1u << (blk & 31u)) - 1u));
      pbyte = uint64_t(rank) * (B / 8u) + (u & (B / 8u - 1u));
    }
    if (coded) {
      const uint32_t p0 = in[g.plane + pbyte];
      const uint32_t p1 = in[g.plane + g.plane_bytes + pbyte];
      const uint32_t p2 = in[g.plane + 2u * g.plane_bytes + pbyte];
      const uint32_t vmask = (valid == 8u) ? 0xFFu : ((1u << valid) - 1u);
      const uint2 codes = codes_from_planes(p0, p1, p2);
      ev[j] = make_uint2(exps_from_codes(codes.x, e0), exps_from_codes(codes.y, e0));
      emask[j] = ~(p0 | p1 | p2) & vmask;
      cnt[j] = __popc(emask[j]);
    } else {
      ev[j] = load_bytes8(cache + start + 8ull * u, valid);
    }
  }
  const uint32_t nesc = chunk_escape_scan(cnt, base, s_tot);
  if (g.esc + pad128(nesc) != end) {
    if (tid == 0) err_slots[c] = uint32_t(CIERA_ERR_FORMAT);
    return;  // uniform: every thread sees the same nesc
  }
#pragma unroll
  for (uint32_t j = 0; j < kUnitsPerThread; j++) {
    const uint32_t u = j * kThreads + tid;
    if (u >= nunits) continue;
    const uint32_t valid = min(8u, nc - 8u * u);
    uint2 e = ev[j];
    uint32_t em = emask[j];
    uint64_t at = g.esc + base[j];
    while (em) {
      const uint32_t k = __builtin_ctz(em);
      em &= em - 1u;
      e = set_byte(e, k, in[at++]);
    }
    store_unit(y, start + 8ull * u, valid, unit_join(smv[j], e));
    if (kCiera) {
      const uint32_t blk = (8u * u) >> log2B;
      if ((s_bits[blk >> 5] >> (blk & 31u)) & 1u) store_bytes8(cache + start + 8ull * u, valid, e);
    }
  }
  if (tid == 0) err_slots[c] = 0u;
}

// ------------------------------------------------------------------ host side
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0u; }

bool valid_block(uint32_t B) { return B >= 64u && B <= kChunk && (B & (B - 1u)) == 0u; }

uint32_t log2u(uint32_t v) {
  uint32_t l = 0;
  while ((1u << l) < v) l++;
  return l;
}

uint64_t max_size(uint64_t n, uint32_t B) {
  const uint64_t nchunks = cdiv(n, kChunk);
  const uint64_t full = n / kChunk;
  const uint64_t rem = n % kChunk;
  auto chunk_max = [B](uint64_t nc) -> uint64_t {
    uint64_t s = 2u * pad128(nc);  // sign+mantissa and worst-case escapes
    if (B) {
      const uint64_t nb = cdiv(nc, B);
      s += pad128(cdiv(nb, 8u)) + 3u * pad128(nb * B / 8u);
    } else {
      s += 3u * pad128(cdiv(nc, 8u));
    }
    return s;
  };
  return table_end(nchunks) + full * chunk_max(kChunk) + (rem ? chunk_max(rem) : 0u);
}

ciera_status launch_status() {
  return hipGetLastError() == hipSuccess ? CIERA_OK : CIERA_ERR_HIP;
}

ciera_status encode_impl(const void* d_x, uint64_t n, uint32_t B, uint8_t* d_cache, void* d_out,
                         uint64_t out_capacity, void* d_ws, uint64_t ws_bytes, uint64_t* d_out_size,
                         int e0_override, hipStream_t stream) {
  const bool ciera = B != 0u;
  if (n > kMaxN) return CIERA_ERR_ARG;
  if (ciera && !valid_block(B)) return CIERA_ERR_ARG;
  if (e0_override < -1 || e0_override > int(kMaxE0)) return CIERA_ERR_ARG;
  if (!d_out || !d_ws || !d_out_size || !aligned16(d_out) || !aligned16(d_ws)) return CIERA_ERR_ARG;
  if ((reinterpret_cast<uintptr_t>(d_out_size) & 7u) != 0u) return CIERA_ERR_ARG;
  if (n > 0 && (!d_x || !aligned16(d_x))) return CIERA_ERR_ARG;
  if (ciera && n > 0 && (!d_cache || !aligned16(d_cache))) return CIERA_ERR_ARG;
  if (out_capacity < max_size(n, B)) return CIERA_ERR_CAPACITY;
  const uint64_t nchunks = cdiv(n, kChunk);
  if (ws_bytes < ws_layout(nchunks).total) return CIERA_ERR_WORKSPACE;
  const Ws ws = ws_bind(d_ws, nchunks);
  const uint32_t lb = ciera ? log2u(B) : 0u;
  const uint16_t* x = static_cast<const uint16_t*>(d_x);
  uint8_t* out = static_cast<uint8_t*>(d_out);
  (void)hipGetLastError();
  if (nchunks) {
    if (ciera)
      hipLaunchKernelGGL(k_stats<true>, dim3(uint32_t(nchunks)), dim3(kThreads), 0, stream, x, n, d_cache, lb, ws);
    else
      hipLaunchKernelGGL(k_stats<false>, dim3(uint32_t(nchunks)), dim3(kThreads), 0, stream, x, n, nullptr, 0u, ws);
  }
  hipLaunchKernelGGL(k_plan, dim3(1), dim3(kThreads), 0, stream, n, nchunks, B, e0_override, out, d_out_size, ws);
  if (nchunks) {
    if (ciera)
      hipLaunchKernelGGL(k_write<true>, dim3(uint32_t(nchunks)), dim3(kThreads), 0, stream, x, n, nchunks, lb, out,
                         d_out_size, ws);
    else
      hipLaunchKernelGGL(k_write<false>, dim3(uint32_t(nchunks)), dim3(kThreads), 0, stream, x, n, nchunks, 0u,
                         out, d_out_size, ws);
  }
  return launch_status();
}

ciera_status decode_impl(const void* d_in, uint64_t in_size, void* d_y, uint64_t n, uint32_t B,
                         uint8_t* d_cache, void* d_ws, uint64_t ws_bytes, hipStream_t stream) {
  const bool ciera = B != 0u;
  if (n > kMaxN) return CIERA_ERR_ARG;
  if (ciera && !valid_block(B)) return CIERA_ERR_ARG;
  if (!d_in || !d_ws || !aligned16(d_in) || !aligned16(d_ws)) return CIERA_ERR_ARG;
  if (n > 0 && (!d_y || !aligned16(d_y))) return CIERA_ERR_ARG;
  if (ciera && n > 0 && (!d_cache || !aligned16(d_cache))) return CIERA_ERR_ARG;
  const uint64_t nchunks = cdiv(n, kChunk);
  if (ws_bytes < ws_layout(nchunks).total) return CIERA_ERR_WORKSPACE;
  const Ws ws = ws_bind(d_ws, nchunks);
  const uint32_t grid = uint32_t(nchunks ? nchunks : 1u);
  const uint8_t* in = static_cast<const uint8_t*>(d_in);
  uint16_t* y = static_cast<uint16_t*>(d_y);
  (void)hipGetLastError();
  if (ciera)
    hipLaunchKernelGGL(k_decode<true>, dim3(grid), dim3(kThreads), 0, stream, in, in_size, y, n, nchunks, log2u(B),
                       d_cache, &ws.ctrl->n_err_slots, ws.err);
  else
    hipLaunchKernelGGL(k_decode<false>, dim3(grid), dim3(kThreads), 0, stream, in, in_size, y, n, nchunks, 0u,
                       nullptr, &ws.ctrl->n_err_slots, ws.err);
  return launch_status();
}

}  // namespace

extern "C" {

uint64_t zip3_max_encoded_size(uint64_t n) { return n > kMaxN ? 0u : max_size(n, 0u); }

uint64_t ciera_max_encoded_size(uint64_t n, uint32_t B) {
  return (n > kMaxN || !valid_block(B)) ? 0u : max_size(n, B);
}

uint64_t zip3_workspace_size(uint64_t n) { return n > kMaxN ? 0u : ws_layout(cdiv(n, kChunk)).total; }

uint64_t ciera_workspace_size(uint64_t n, uint32_t B) {
  return (n > kMaxN || !valid_block(B)) ? 0u : ws_layout(cdiv(n, kChunk)).total;
}

ciera_status zip3_encode(const void* d_x, uint64_t n, void* d_out, uint64_t out_capacity, void* d_ws,
                         uint64_t ws_bytes, uint64_t* d_out_size, hipStream_t stream) {
  return encode_impl(d_x, n, 0u, nullptr, d_out, out_capacity, d_ws, ws_bytes, d_out_size, -1, stream);
}

ciera_status zip3_encode_ex(const void* d_x, uint64_t n, void* d_out, uint64_t out_capacity, void* d_ws,
                            uint64_t ws_bytes, uint64_t* d_out_size, int e0_override, hipStream_t stream) {
  return encode_impl(d_x, n, 0u, nullptr, d_out, out_capacity, d_ws, ws_bytes, d_out_size, e0_override, stream);
}

ciera_status zip3_decode(const void* d_in, uint64_t in_size, void* d_y, uint64_t n, void* d_ws,
                         uint64_t ws_bytes, hipStream_t stream) {
  return decode_impl(d_in, in_size, d_y, n, 0u, nullptr, d_ws, ws_bytes, stream);
}

ciera_status ciera_encode(const void* d_x, uint64_t n, uint32_t B, uint8_t* d_prev_exp, void* d_out,
                          uint64_t out_capacity, void* d_ws, uint64_t ws_bytes, uint64_t* d_out_size,
                          hipStream_t stream) {
  if (B == 0u) return CIERA_ERR_ARG;
  return encode_impl(d_x, n, B, d_prev_exp, d_out, out_capacity, d_ws, ws_bytes, d_out_size, -1, stream);
}

ciera_status ciera_encode_ex(const void* d_x, uint64_t n, uint32_t B, uint8_t* d_prev_exp, void* d_out,
                             uint64_t out_capacity, void* d_ws, uint64_t ws_bytes, uint64_t* d_out_size,
                             int e0_override, hipStream_t stream) {
  if (B == 0u) return CIERA_ERR_ARG;
  return encode_impl(d_x, n, B, d_prev_exp, d_out, out_capacity, d_ws, ws_bytes, d_out_size, e0_override,
                     stream);
}

ciera_status ciera_decode(const void* d_in, uint64_t in_size, void* d_y, uint64_t n, uint32_t B,
                          uint8_t* d_prev_exp, void* d_ws, uint64_t ws_bytes, hipStream_t stream) {
  if (B == 0u) return CIERA_ERR_ARG;
  return decode_impl(d_in, in_size, d_y, n, B, d_prev_exp, d_ws, ws_bytes, stream);
}

ciera_status ciera_read_error(const void* d_ws, hipStream_t stream) {
  if (!d_ws) return CIERA_ERR_ARG;
  const Ctrl* ctrl = static_cast<const Ctrl*>(d_ws);
  uint64_t slots = 0;
  if (hipMemcpyAsync(&slots, &ctrl->n_err_slots, sizeof(slots), hipMemcpyDeviceToHost, stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess)
    return CIERA_ERR_HIP;
  if (slots == 0u) return CIERA_OK;
  if (slots > cdiv(kMaxN, kChunk)) return CIERA_ERR_INTERNAL;
  const uint32_t* err = reinterpret_cast<const uint32_t*>(static_cast<const uint8_t*>(d_ws) + sizeof(Ctrl));
  uint32_t worst = 0;
  uint32_t buf[4096];
  for (uint64_t at = 0; at < slots; at += 4096u) {
    const uint64_t cnt = (slots - at < 4096u) ? slots - at : 4096u;
    if (hipMemcpyAsync(buf, err + at, cnt * 4u, hipMemcpyDeviceToHost, stream) != hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess)
      return CIERA_ERR_HIP;
    for (uint64_t i = 0; i < cnt; i++)
      if (buf[i] > worst) worst = buf[i];
  }
  return ciera_status(worst);
}

const char* ciera_status_string(ciera_status status) {
  switch (status) {
    case CIERA_OK: return "ok";
    case CIERA_ERR_ARG: return "invalid argument";
    case CIERA_ERR_CAPACITY: return "output capacity too small";
    case CIERA_ERR_WORKSPACE: return "workspace too small";
    case CIERA_ERR_HIP: return "HIP runtime error";
    case CIERA_ERR_FORMAT: return "malformed stream";
    case CIERA_ERR_INTERNAL: return "internal error";
    default: return "unknown status";
  }
}

}  // extern "C"
