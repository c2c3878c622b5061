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

// Eight BF16 patterns of unit u (first value index `first`), `cnt` of them
// real; the rest read as zero.
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

__device__ inline uint64_t load_bytes8(const uint8_t* __restrict__ p, uint32_t cnt) {
  if (cnt == 8u) return *reinterpret_cast<const uint64_t*>(p);
  uint64_t v = 0;
  for (uint32_t k = 0; k < cnt; k++) v |= uint64_t(p[k]) << (8u * k);
  return v;
}

__device__ inline void store_bytes8(uint8_t* __restrict__ p, uint32_t cnt, uint64_t v) {
  if (cnt == 8u) {
    *reinterpret_cast<uint64_t*>(p) = v;
  } else {
    for (uint32_t k = 0; k < cnt; k++) p[k] = uint8_t(v >> (8u * k));
  }
}

__device__ inline uint32_t value_bits(const Unit& u, uint32_t k) {
  return (u.w[k >> 1] >> (16u * (k & 1u))) & 0xFFFFu;
}

// Exponent fields of the unit's 8 values, byte k = exponent of value k.
__device__ inline uint64_t unit_exponents(const Unit& u) {
  uint64_t e = 0;
#pragma unroll
  for (uint32_t k = 0; k < 8u; k++) e |= uint64_t((value_bits(u, k) >> 7) & 0xFFu) << (8u * k);
  return e;
}

// Sign+mantissa bytes, byte k = (sign << 7) | mantissa of value k.
__device__ inline uint64_t unit_sm(const Unit& u) {
  uint64_t s = 0;
#pragma unroll
  for (uint32_t k = 0; k < 8u; k++) {
    const uint32_t v = value_bits(u, k);
    s |= uint64_t(((v >> 8) & 0x80u) | (v & 0x7Fu)) << (8u * k);
  }
  return s;
}

// Exact FP64 value of a finite BF16 pattern, built from its integer fields.
__device__ inline double bf16_value(uint32_t v) {
  const uint32_t e = (v >> 7) & 0xFFu;
  const uint32_t m = v & 0x7Fu;
  const double mag = e ? ldexp(double(128u + m), int(e) - 134) : ldexp(double(m), -133);
  return (v & 0x8000u) ? -mag : mag;
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

__device__ inline uint32_t wave_sum_u32(uint32_t v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
  return v;
}

// Escape positions: each thread holds kUnitsPerThread counts (one per unit,
// 0..8), units ordered (j, wave, lane).  On return base[j] is the number of
// escapes in all earlier units of the chunk and the function returns the
// chunk total.  Needs a barrier-safe call by every thread of the workgroup.
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
  const double shift = (((first >> 7) & 0xFFu) != 0xFFu) ? bf16_value(first) : 0.0;
  __syncthreads();

  double s1 = 0.0, s2 = 0.0;
  uint32_t nf = 0;
#pragma unroll
  for (uint32_t j = 0; j < kUnitsPerThread; j++) {
    const uint32_t u = j * kThreads + tid;
    if (u >= nunits) break;
    const uint32_t cnt = min(8u, nc - 8u * u);
    const uint64_t at = start + 8ull * u;
    const Unit v = load_unit(x, at, cnt);
#pragma unroll
    for (uint32_t k = 0; k < 8u; k++) {
      const uint32_t b = value_bits(v, k);
      if (k < cnt && ((b >> 7) & 0xFFu) != 0xFFu) {
        const double d = bf16_value(b) - shift;
        s1 += d;
        s2 = fma(d, d, s2);
        nf++;
      }
    }
    if (kCiera) {
      const uint64_t e = unit_exponents(v);
      const uint64_t old = load_bytes8(cache + at, cnt);
      const uint64_t keep = (cnt == 8u) ? ~0ull : ((1ull << (8u * cnt)) - 1u);
      if ((e ^ old) & keep) {
        store_bytes8(cache + at, cnt, e);
        const uint32_t blk = (8u * u) >> log2B;
        atomicOr(&s_bits[blk >> 5], 1u << (blk & 31u));
      }
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
__device__ inline uint32_t window_base(double var, uint64_t nf) {
  if (nf < 2u || !(var > 0.0)) return 0u;
  uint32_t e0 = 0u;
  for (int k = -127; k <= 122; k++)
    if (var >= ldexp(kK0, 2 * k)) e0 = uint32_t(127 + k);
  return e0;
}

__global__ __launch_bounds__(kThreads) void k_plan(uint64_t n, uint64_t nchunks, uint32_t B, int e0_override,
                                                   uint8_t* __restrict__ out, uint64_t* __restrict__ out_size,
                                                   Ws ws) {
  __shared__ double s_s1[kThreads], s_s2[kThreads];
  __shared__ uint64_t s_nf[kThreads], s_nch[kThreads];
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
  s_s1[tid] = a;
  s_s2[tid] = b;
  s_nf[tid] = m;
  s_nch[tid] = q;
  __syncthreads();
  for (uint32_t h = kThreads / 2u; h >= 1u; h >>= 1) {
    if (tid < h) {
      s_s1[tid] += s_s1[tid + h];
      s_s2[tid] += s_s2[tid + h];
      s_nf[tid] += s_nf[tid + h];
      s_nch[tid] += s_nch[tid + h];
    }
    __syncthreads();
  }
  uint64_t* table = reinterpret_cast<uint64_t*>(out + kHeader);
  const uint64_t base = table_end(nchunks);
  // zero the table's padding words (entries past nchunks)
  for (uint64_t i = nchunks + 1u + tid; i < (base - kHeader) / 8u; i += kThreads) table[i] = 0u;
  if (tid == 0) {
    const uint64_t nf = s_nf[0];
    double var = 0.0;
    if (nf >= 2u) {
      var = (s_s2[0] - s_s1[0] * s_s1[0] / double(nf)) / double(nf - 1u);
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
    h[5] = s_nch[0];
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

  // Load the chunk and derive per-unit fields.
  Unit v[kUnitsPerThread];
  uint32_t cnt[kUnitsPerThread], base[kUnitsPerThread];
  uint32_t planes[kUnitsPerThread];  // p0 | p1 << 8 | p2 << 16, escape mask << 24
#pragma unroll
  for (uint32_t j = 0; j < kUnitsPerThread; j++) {
    const uint32_t u = j * kThreads + tid;
    cnt[j] = 0u;
    planes[j] = 0u;
    if (u < nunits) {
      const uint32_t valid = min(8u, nc - 8u * u);
      v[j] = load_unit(x, start + 8ull * u, valid);
      bool coded = true;
      if (kCiera) {
        const uint32_t blk = (8u * u) >> log2B;
        coded = (s_bits[blk >> 5] >> (blk & 31u)) & 1u;
      }
      if (coded) {
        const uint32_t vmask = (valid == 8u) ? 0xFFu : ((1u << valid) - 1u);
        uint32_t p0 = 0, p1 = 0, p2 = 0, em = 0;
#pragma unroll
        for (uint32_t k = 0; k < 8u; k++) {
          const uint32_t e = (value_bits(v[j], k) >> 7) & 0xFFu;
          const uint32_t d = e - e0;
          const uint32_t code = (d <= 6u) ? d + 1u : 0u;
          p0 |= (code & 1u) << k;
          p1 |= ((code >> 1) & 1u) << k;
          p2 |= ((code >> 2) & 1u) << k;
          em |= uint32_t(code == 0u) << k;
        }
        p0 &= vmask;
        p1 &= vmask;
        p2 &= vmask;
        em &= vmask;
        planes[j] = p0 | (p1 << 8) | (p2 << 16) | (em << 24) | 0u;
        cnt[j] = __popc(em);
      }
    } else {
      v[j].w[0] = v[j].w[1] = v[j].w[2] = v[j].w[3] = 0u;
    }
  }
  const uint32_t nesc = chunk_escape_scan(cnt, base, s_tot);

  // Chunk size and offset (decoupled look-back over earlier chunks).
  const uint64_t size = pad128(nc) + (kCiera ? 128u : 0u) +
                        3u * pad128(kCiera ? uint64_t(nch) * B / 8u : cdiv(nc, 8u)) + pad128(nesc);
  if (tid == 0) {
    uint32_t err = 0u;
    atomicAdd(reinterpret_cast<unsigned long long*>(&ws.ctrl->esc_total), (unsigned long long)nesc);
    uint64_t prefix = 0;
    if (c == 0u) {
      __hip_atomic_store(&ws.status[c], kFlagInclusive | size, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      __hip_atomic_store(&ws.status[c], kFlagAggregate | size, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
      int64_t k = int64_t(c) - 1;
      uint32_t spins = 0;
      while (k >= 0) {
        const uint64_t s = __hip_atomic_load(&ws.status[k], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
        if ((s & ~kValueMask) == 0u) {
          if (++spins > kSpinLimit) {
            err = CIERA_ERR_INTERNAL;
            break;
          }
          __builtin_amdgcn_s_sleep(1);
          continue;
        }
        prefix += s & kValueMask;
        if ((s & ~kValueMask) == kFlagInclusive) break;
        k--;
      }
      __hip_atomic_store(&ws.status[c], kFlagInclusive | (prefix + size), __ATOMIC_RELEASE,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
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
  __syncthreads();
  if (s_err) return;  // uniform; the error word tells the caller
  const ChunkGeom g = chunk_geom(s_begin, nc, kCiera, nch, B);

  // Write sections.
#pragma unroll
  for (uint32_t j = 0; j < kUnitsPerThread; j++) {
    const uint32_t u = j * kThreads + tid;
    if (u >= nunits) continue;
    *reinterpret_cast<uint64_t*>(out + g.sm + 8ull * u) = unit_sm(v[j]);
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
        const uint64_t e = unit_exponents(v[j]);
        uint64_t at = g.esc + base[j];
        while (em) {
          const uint32_t k = __builtin_ctz(em);
          em &= em - 1u;
          out[at++] = uint8_t(e >> (8u * k));
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

  uint64_t smv[kUnitsPerThread], ev[kUnitsPerThread];
  uint32_t cnt[kUnitsPerThread], base[kUnitsPerThread], emask[kUnitsPerThread];
#pragma unroll
  for (uint32_t j = 0; j < kUnitsPerThread; j++) {
    const uint32_t u = j * kThreads + tid;
    cnt[j] = 0u;
    emask[j] = 0u;
    smv[j] = 0u;
    ev[j] = 0u;
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
      uint64_t e = 0;
#pragma unroll
      for (uint32_t k = 0; k < 8u; k++) {
        const uint32_t code = ((p0 >> k) & 1u) | (((p1 >> k) & 1u) << 1) | (((p2 >> k) & 1u) << 2);
        e |= uint64_t(code ? e0 + code - 1u : 0u) << (8u * k);
      }
      ev[j] = e;
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
    uint64_t e = ev[j];
    uint32_t em = emask[j];
    uint64_t at = g.esc + base[j];
    while (em) {
      const uint32_t k = __builtin_ctz(em);
      em &= em - 1u;
      e |= uint64_t(in[at++]) << (8u * k);
    }
    Unit o;
#pragma unroll
    for (uint32_t k2 = 0; k2 < 4u; k2++) {
      uint32_t w = 0;
#pragma unroll
      for (uint32_t h = 0; h < 2u; h++) {
        const uint32_t k = 2u * k2 + h;
        const uint32_t sm = uint32_t(smv[j] >> (8u * k)) & 0xFFu;
        const uint32_t ex = uint32_t(e >> (8u * k)) & 0xFFu;
        w |= (((sm & 0x80u) << 8) | (ex << 7) | (sm & 0x7Fu)) << (16u * h);
      }
      o.w[k2] = w;
    }
    store_unit(y, start + 8ull * u, valid, o);
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
