// ciera.hip -- HIP kernels and C ABI of the lossless BF16 codec, gfx950.
//
// Encode is four kernels on the caller's stream:
//   k_stats   one workgroup per quarter chunk ("part", 16,384 values), one
//             pass over the input: FP64 partial sums for the tensor's
//             variance (ZipCCL research digest, section 3.1: sigma from one
//             standard-deviation pass); in ciera mode the changed-block bits
//             against the sender's exponent cache and the cache update (CIERA
//             page, section 3.1); and an exponent histogram of the values to
//             be coded.
//   k_sums    per planning group (a range of chunks), the parts' partial
//             sums added in a fixed order.
//   k_plan    the same groups (up to 256): add the groups' sums in a fixed
//             order and pick the window base E0 (integer nearest x_opt =
//             log2 sigma + 0.5 log2(14 ln2 / 16383), digest section 3.1,
//             evaluated as var >= K0 4^k); each part's escape count is its
//             number of coded values outside [E0, E0+6], read off the
//             histogram, so chunk sizes follow exactly and a scan turns them
//             into the chunk table (the size exchange of the digest's
//             Figure 1, done on one GPU).
//   k_write   one workgroup per part, no synchronisation with any other:
//             splits values into sign+mantissa bytes and 3-bit codes and
//             writes the 128-byte-aligned sections at offsets k_plan fixed
//             (digest, section 3.1 last paragraph).
// A tensor of at most 16 chunks is two kernels: k_stats, then k_write,
// which plans for itself.
// Decode is one kernel, k_decode, one workgroup per part; parts are
// independent because the chunk table holds every chunk offset and the
// escape index each part's first escape.  k_decode_batch runs the same
// workgroups for several streams of one size in one launch.
// The single-read encodes (window base given) are k_prep1 + k_write1; the
// rANS modes k_stats + k_rans_enc + k_rans_finish, and k_rans_dec.  The
// speculative encodes (window base hinted) run k_prep1 + k_write1 with the
// variance sums, k_sums and k_check, then k_stats (recorded change bits),
// k_plan and k_write, which return at once when the hint was right.
//
// Work mapping: a "unit" is 8 consecutive values (one 16-byte load).  A chunk
// has 8192 units.  In k_stats, k_write and k_decode part h covers units
// [2048h, 2048h + 2048) and thread t of its 256 handles unit 2048h + 256j + t
// (j = 0..7), so each wave instruction moves 1 KiB of contiguous input.  For
// tensors of at most 16 chunks (k_stats, k_write) or 32 (k_decode) each part
// is split into four slices of 512 units, one workgroup each, so that a
// shard-sized tensor spreads over every CU.
// Blocks (B >= 64) never split a unit, and chunks never split a block.  All
// data movement is integer: sign, NaN payloads, subnormals and -0 never pass
// through floating-point registers.
// Loads: a thread issues all loads of a full range before it uses any, and
// none sits under a per-lane condition: the compiler would copy such a
// load's result into place only after waiting for every load issued before
// it, one round trip per load.  A lane that needs no data (a unit of a
// changed block in the decoders) reads the chunk's first bytes instead, one
// line for all such lanes of the wave.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include <atomic>
#include <type_traits>
#include <mutex>
#include <vector>

#include "ciera.h"

namespace {

constexpr uint32_t kChunk = 65536u;
constexpr uint32_t kThreads = 1024u;  // k_prep1
constexpr uint32_t kUnitsPerChunk = kChunk / 8u;
constexpr uint32_t kBitmapWords = 32u;  // 1024 blocks per chunk at B = 64
constexpr uint64_t kMaxN = 1ull << 40;
constexpr uint64_t kHeader = 128u;
constexpr uint32_t kMaxE0 = 249u;
constexpr uint32_t kBadE0 = ~0u;  // control-block E0 of a call whose given window base is out of range
// 16383 / (28 ln 2) as a double: the variance threshold of window base k is
// kK0 * 4^k.
constexpr double kK0 = 0x1.a610ca4a234eep+9;

// Parts: k_write and k_decode run kParts workgroups of kPartThreads threads
// per chunk, kUPT units per thread.
constexpr uint32_t kParts = 4u;
constexpr uint32_t kPartThreads = 256u;
constexpr uint32_t kPartWaves = kPartThreads / 64u;
constexpr uint32_t kUPT = 8u;
constexpr uint32_t kPartUnits = kPartThreads * kUPT;  // 2048 units = 16384 values
static_assert(kPartUnits * kParts == kUnitsPerChunk, "parts tile a chunk");
static_assert(kUPT * kPartWaves <= 64u, "one scan entry per lane");
constexpr uint32_t kStage = kPartUnits + 16u;  // LDS bytes per staged plane
constexpr uint32_t kPartEscStage = 16384u + 32u;  // a part's escapes (at most its 16,384 values) staged in LDS
constexpr uint32_t kBins = 256u;               // exponent histogram bins
constexpr uint32_t kHistCopies = 16u;          // interleaved LDS copies (by lane) to spread atomics
static_assert(kPartThreads == kBins, "k_stats stores one bin per thread");
constexpr uint32_t kPartValues = kPartUnits * 8u;                 // 16384
constexpr uint32_t kPartBitmapWords = kBitmapWords / kParts;      // 8: one bit per block at B = 64
static_assert(kPartBitmapWords * 32u * 64u == kPartValues, "a part's blocks fit its bitmap words");

__host__ __device__ inline uint64_t pad128(uint64_t v) { return (v + 127u) & ~uint64_t(127); }
__host__ __device__ inline uint64_t cdiv(uint64_t a, uint64_t b) { return (a + b - 1u) / b; }
// After the header: the chunk table (nchunks + 1 absolute u64 offsets), then
// the escape index (per chunk one u64 of four u16: the escapes among the
// chunk's values before value 0, 16384, 32768 and 49152 of the chunk, i.e.
// before each part), zero-padded to 128 bytes.  The index lets every part
// of a chunk find its first escape without reading the parts before it.
__host__ __device__ inline uint64_t table_end(uint64_t nchunks) {
  return kHeader + pad128(8u * (nchunks + 1u) + 8u * nchunks);
}
static_assert(kParts == 4u, "one u64 of four u16 escape counts per chunk");
// Largest stream bytes of a chunk of nc values (B = 0: zip3): every value
// escapes and, in ciera mode, every block changed.
__host__ __device__ inline uint64_t chunk_max_bytes(uint64_t nc, uint32_t B) {
  uint64_t s = 2u * pad128(nc);  // sign+mantissa and escapes
  if (B) {
    const uint64_t nb = cdiv(nc, B);
    s += pad128(cdiv(nb, 8u)) + 3u * pad128(nb * B / 8u);
  } else {
    s += 3u * pad128(cdiv(nc, 8u));
  }
  return s;
}

// Every wait of one workgroup on another is bounded: it gives up after this
// many polls (seconds of GPU time; it ends only a wait that would not end).
constexpr uint32_t kSpinLimit = 1u << 22;

// Workspace: control block, error words, per-part partial sums and bitmap
// words, exponent histograms of the parts, per-part escape offsets
// and per-chunk escape totals, and the look-back words of the single-read
// encode.
struct Ctrl {
  uint32_t e0;
  uint32_t plan_fail;  // set by a k_plan workgroup whose wait did not end
  uint64_t n_err_slots;
  uint64_t done_esc;  // single-read encode: chunks finished << 40 | their escapes
  uint64_t done_nch;  // single-read ciera encode: the finished chunks' changed blocks
  uint32_t spec;       // speculative encode: kSpecHit once k_check found the hinted window right
  uint32_t spec_fail;  // speculative encode: set by a write workgroup that did not finish the stream
  uint64_t reserved[27];
};
static_assert(sizeof(Ctrl) == 256, "control block is 256 bytes");

struct Partial {
  double s1;
  double s2;
  uint32_t nf;
  uint32_t nch;
  uint32_t coded;  // values the part codes (all of them in zip3 mode)
  uint32_t pad;
};

// k_sums and k_plan run as up to kPlanMaxGroups workgroups, each over a
// contiguous range of chunks.  k_sums stores each group's variance sums in
// its slot; k_plan publishes each group's stream bytes, escapes and changed
// blocks there, each in a word that k_stats cleared (not ready).
constexpr uint32_t kPlanThreads = 256u;
constexpr uint32_t kPlanWaves = kPlanThreads / 64u;
constexpr uint32_t kPlanMaxGroups = kPlanThreads;  // one slot per thread in the waits
constexpr uint32_t kPlanMinChunks = 16u;           // chunks per group, unless that needs too many groups
constexpr uint64_t kSlotReady = 1ull << 63;        // set in the count words

struct PlanSlot {
  uint64_t s1, s2;            // FP64 bit patterns of the group's variance sums (k_sums)
  uint64_t nf;                // finite values (k_sums)
  uint64_t bytes, esc, nch;   // kSlotReady | the group's stream bytes, escapes, changed blocks (k_plan)
  uint64_t pad[2];
};
static_assert(sizeof(PlanSlot) == 64, "plan slot is 64 bytes");

// Single-read look-back: each chunk's status word and its four part counts
// sit on a 128-byte line of their own (strides in words).  Neighbouring
// chunks are written and polled by workgroups on different XCDs; when they
// shared lines, the line moved between the L2s on every write and the
// single-read encode of a 64M-value tensor took a quarter longer.
constexpr uint32_t kCstatStride = 16u;   // u64 words
constexpr uint32_t kPcountStride = 32u;  // u32 words
// rANS encode: the look-back word of each part, likewise on a line of its own.
constexpr uint32_t kRstatStride = 16u;   // u64 words

struct WsLayout {
  uint64_t err, partial, bitmap, hist, partesc, chunkesc, pcount, cstat, plan, phash, total;
};

// Decoding tensors of at most kSliceChunks chunks: kSlices workgroups per
// part, each decoding a slice of it (two units per thread instead of eight),
// so that a shard-sized tensor keeps every CU busy instead of one per part.
constexpr uint32_t kSlices = 4u;
constexpr uint64_t kSliceChunks = 32u;
static_assert(kUPT % kSlices == 0u && (kUPT / kSlices) % 2u == 0u, "unit pairs per thread in a slice");

// Exponent histograms: per part one row of kBins u16 counts (a part holds at
// most 16384 values) of its coded values by exponent field, rows in part
// order, so that each part writes whole 128-byte lines.

__host__ __device__ inline uint64_t align256(uint64_t v) { return (v + 255u) & ~uint64_t(255); }

__host__ inline WsLayout ws_layout(uint64_t nchunks) {
  WsLayout l;
  const uint64_t slots = nchunks ? nchunks : 1u;
  l.err = sizeof(Ctrl);
  // one error word per workgroup; per-part records of k_stats, per slice for small tensors
  const uint64_t recs = kParts * slots * (slots <= kSliceChunks ? kSlices : 1u);
  l.partial = align256(l.err + 4u * recs);
  l.bitmap = align256(l.partial + sizeof(Partial) * recs);
  l.hist = align256(l.bitmap + 4u * kPartBitmapWords * recs);
  l.partesc = align256(l.hist + 2u * kBins * recs);
  l.chunkesc = align256(l.partesc + 4u * kParts * slots);
  l.pcount = align256(l.chunkesc + 4u * slots);
  l.cstat = align256(l.pcount + 4u * kPcountStride * slots);
  l.plan = align256(l.cstat + 8u * kCstatStride * slots);
  l.phash = align256(l.plan + sizeof(PlanSlot) * kPlanMaxGroups);
  l.total = align256(l.phash + 16u * kParts * slots);
  return l;
}

struct Ws {
  Ctrl* ctrl;
  uint32_t* err;        // one word per workgroup of k_write / k_decode
  Partial* partial;     // per part
  uint32_t* bitmap;     // kPartBitmapWords per part
  uint16_t* hist;       // kBins u16 per part
  uint32_t* partesc;    // escapes before each part within its chunk
  uint32_t* chunkesc;   // escapes per chunk
  // single-read encode: look-back words
  uint32_t* pcount;     // per part, kPcountStride per chunk: kPartReady | escapes of the part
  uint64_t* cstat;      // per chunk, kCstatStride apart: flag | stream bytes (inclusive prefix)
  PlanSlot* plan;       // per k_plan workgroup
  uint64_t* phash;      // hash sender, blocks larger than a part: the part's two partial hashes
  // rANS modes only (null otherwise): per part a look-back word, its coded
  // count and changed blocks, and a scratch slot for its payload
  uint64_t* rstat;
  uint64_t* rinfo;
  uint8_t* rslot;
  uint32_t spin_limit;  // polls before a wait gives up (kSpinLimit unless a test lowers it)
  uint32_t ss;          // k_stats records per part: 1, or kSlices (one per slice) for self-planned tensors
  const uint8_t* e0_src;  // self-planned encode with a known window base: its byte in device memory, else null
  uint32_t spec;          // a speculative encode's fallback launch: do nothing if ctrl->spec == kSpecHit
};
constexpr uint32_t kSpecHit = 1u;

// The bound the next calls pass to their kernels (ciera_set_wait_limit).
std::atomic<uint32_t> g_wait_limit{kSpinLimit};

__host__ inline Ws ws_bind(void* base, uint64_t nchunks) {
  const WsLayout l = ws_layout(nchunks);
  uint8_t* b = static_cast<uint8_t*>(base);
  Ws w;
  w.ctrl = reinterpret_cast<Ctrl*>(b);
  w.err = reinterpret_cast<uint32_t*>(b + l.err);
  w.partial = reinterpret_cast<Partial*>(b + l.partial);
  w.bitmap = reinterpret_cast<uint32_t*>(b + l.bitmap);
  w.hist = reinterpret_cast<uint16_t*>(b + l.hist);
  w.partesc = reinterpret_cast<uint32_t*>(b + l.partesc);
  w.chunkesc = reinterpret_cast<uint32_t*>(b + l.chunkesc);
  w.pcount = reinterpret_cast<uint32_t*>(b + l.pcount);
  w.cstat = reinterpret_cast<uint64_t*>(b + l.cstat);
  w.plan = reinterpret_cast<PlanSlot*>(b + l.plan);
  w.phash = reinterpret_cast<uint64_t*>(b + l.phash);
  w.rstat = nullptr;
  w.rinfo = nullptr;
  w.rslot = nullptr;
  w.spin_limit = g_wait_limit.load(std::memory_order_relaxed);
  w.ss = 1u;
  w.e0_src = nullptr;
  w.spec = 0u;
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
    // unrolled so that every index into w is a constant (no private array)
#pragma unroll
    for (uint32_t i = 0; i < 4u; i++) {
      const uint32_t lo = (2u * i < cnt) ? uint32_t(x[first + 2u * i]) : 0u;
      const uint32_t hi = (2u * i + 1u < cnt) ? uint32_t(x[first + 2u * i + 1u]) : 0u;
      u.w[i] = lo | (hi << 16);
    }
  }
  return u;
}

// Decoded values: full units go out as non-temporal 16-byte stores, so that
// the decoder's output does not sit dirty in the MALL (256 MB) and get
// written back while the next kernel streams its own input.
__device__ inline void store_unit(uint16_t* __restrict__ y, uint64_t first, uint32_t cnt, const Unit& u) {
  if (cnt == 8u) {
    typedef unsigned int v4u __attribute__((ext_vector_type(4)));
    const v4u val = {u.w[0], u.w[1], u.w[2], u.w[3]};
    __builtin_nontemporal_store(val, reinterpret_cast<v4u*>(y + first));
  } else {
#pragma unroll
    for (uint32_t i = 0; i < 4u; i++) {
      if (2u * i < cnt) y[first + 2u * i] = uint16_t(u.w[i]);
      if (2u * i + 1u < cnt) y[first + 2u * i + 1u] = uint16_t(u.w[i] >> 16);
    }
  }
}

__device__ inline uint2 load_bytes8(const uint8_t* __restrict__ p, uint32_t cnt) {
  if (cnt == 8u) return *reinterpret_cast<const uint2*>(p);
  uint2 v = make_uint2(0u, 0u);
#pragma unroll
  for (uint32_t k = 0; k < 8u; k++) {
    if (k < cnt) {
      if (k < 4u)
        v.x |= uint32_t(p[k]) << (8u * k);
      else
        v.y |= uint32_t(p[k]) << (8u * (k - 4u));
    }
  }
  return v;
}

__device__ inline void store_bytes8(uint8_t* __restrict__ p, uint32_t cnt, uint2 v) {
  if (cnt == 8u) {
    *reinterpret_cast<uint2*>(p) = v;
  } else {
#pragma unroll
    for (uint32_t k = 0; k < 8u; k++)
      if (k < cnt) p[k] = uint8_t((k < 4u ? v.x : v.y) >> (8u * (k & 3u)));
  }
}

// Cache rewrite by whole lines: m is the wave's ballot of "this lane's unit
// differs from the cache", lane l holding unit u0 + l of 64 consecutive units
// (u0 a multiple of 64), so lanes 16g .. 16g + 15 cover one aligned 128-byte
// line of the cache.  Every lane of a line with some differing unit stores
// its 8 bytes: HBM then sees whole lines.  Stores of only the differing
// units' 8 bytes leave lines partly written; on the 10^9-value stress buffer
// (1 % exponent flips, about 8 % of units differing) the statistics pass
// took 756 us with those and 733 us with whole lines, although it then
// writes 0.72 GB instead of 0.31 GB.
__device__ inline bool line_has_change(uint64_t m) { return ((m >> (lane_id() & 48u)) & 0xFFFFu) != 0u; }

// Bytes sh .. sh + 15 of the 32 bytes p, q (p first), sh < 16.
__device__ inline uint4 shift_bytes(const uint4& p, const uint4& q, uint32_t sh) {
  const uint32_t w[8] = {p.x, p.y, p.z, p.w, q.x, q.y, q.z, q.w};
  const uint32_t r = sh & 3u;
  uint32_t o[4];
  switch (sh >> 2) {  // constant indices in each case (no private array)
    case 0:
#pragma unroll
      for (int i = 0; i < 4; i++) o[i] = __builtin_amdgcn_alignbyte(w[i + 1], w[i], r);
      break;
    case 1:
#pragma unroll
      for (int i = 0; i < 4; i++) o[i] = __builtin_amdgcn_alignbyte(w[i + 2], w[i + 1], r);
      break;
    case 2:
#pragma unroll
      for (int i = 0; i < 4; i++) o[i] = __builtin_amdgcn_alignbyte(w[i + 3], w[i + 2], r);
      break;
    default:
#pragma unroll
      for (int i = 0; i < 4; i++) o[i] = __builtin_amdgcn_alignbyte(w[i + 4], w[i + 3], r);
      break;
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// Copies len bytes from the 16-byte-aligned LDS buffer src to global memory
// at dst with the nthreads threads of a workgroup: aligned 16-byte stores
// over the middle (each built from the two aligned LDS blocks that cover it),
// byte stores only for the unaligned head and tail, so that HBM sees whole
// lines.  src must have 16 readable bytes past len.
__device__ inline void lds_to_global(uint8_t* __restrict__ dst, const uint8_t* src, uint32_t len, uint32_t tid,
                                     uint32_t nthreads) {
  const uint32_t head = min(len, uint32_t((16u - (reinterpret_cast<uintptr_t>(dst) & 15u)) & 15u));
  const uint32_t body = (len - head) / 16u;
  for (uint32_t i = tid; i < head; i += nthreads) dst[i] = src[i];
  for (uint32_t i = tid; i < body; i += nthreads) {
    const uint32_t o = head + 16u * i;
    const uint4* a = reinterpret_cast<const uint4*>(src + (o & ~15u));
    *reinterpret_cast<uint4*>(dst + o) = shift_bytes(a[0], a[1], o & 15u);
  }
  for (uint32_t i = head + 16u * body + tid; i < len; i += nthreads) dst[i] = src[i];
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

// Output values 2i and 2i+1 of a unit from its sign+mantissa bytes (sm) and
// exponent bytes (e), i = 0..3: [s, s', t, t'] with s = sm byte 2i keeps
// mantissa bits 0..6 and, from its copy, the sign at bit 15; the exponent
// bytes placed at bits 0..7 and 16..23 and shifted up by 7 fill bits 7..14.
__device__ inline uint32_t join_word(uint32_t sm, uint32_t e, uint32_t dup_sel, uint32_t exp_sel) {
  return (perm(0u, sm, dup_sel) & 0x807F807Fu) | (perm(0u, e, exp_sel) << 7);
}

__device__ inline Unit unit_join(uint2 sm, uint2 e) {
  Unit o;
  o.w[0] = join_word(sm.x, e.x, 0x01010000u, 0x0C010C00u);
  o.w[1] = join_word(sm.x, e.x, 0x03030202u, 0x0C030C02u);
  o.w[2] = join_word(sm.y, e.y, 0x01010000u, 0x0C010C00u);
  o.w[3] = join_word(sm.y, e.y, 0x03030202u, 0x0C030C02u);
  return o;
}

__device__ inline uint32_t byte_of(uint2 v, uint32_t k) { return ((k < 4u ? v.x : v.y) >> (8u * (k & 3u))) & 0xFFu; }

// Inclusive prefix sum over the 64 lanes of a wave with DPP: shifts by 1, 2,
// 4 and 8 within each 16-lane row, then row 0's total into row 1 and row 2's
// into row 3, then lane 31's running total into rows 2 and 3.
__device__ inline uint32_t wave_incl_scan(uint32_t v) {
  v += __builtin_amdgcn_update_dpp(0u, v, 0x111, 0xF, 0xF, true);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0u, v, 0x112, 0xF, 0xF, true);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0u, v, 0x114, 0xF, 0xF, true);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0u, v, 0x118, 0xF, 0xF, true);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0u, v, 0x142, 0xA, 0xF, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0u, v, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return v;
}

// A 64-bit value from the lane a DPP control selects (0 where it selects none
// or the row is masked off), moved as two 32-bit halves.
template <int kCtrl, int kRowMask, bool kBound>
__device__ inline uint64_t dpp64(uint64_t v) {
  const uint32_t lo = __builtin_amdgcn_update_dpp(0u, uint32_t(v), kCtrl, kRowMask, 0xF, kBound);
  const uint32_t hi = __builtin_amdgcn_update_dpp(0u, uint32_t(v >> 32), kCtrl, kRowMask, 0xF, kBound);
  return (uint64_t(hi) << 32) | lo;
}

__device__ inline uint64_t wave_incl_scan_u64(uint64_t v) {
  v += dpp64<0x111, 0xF, true>(v);
  v += dpp64<0x112, 0xF, true>(v);
  v += dpp64<0x114, 0xF, true>(v);
  v += dpp64<0x118, 0xF, true>(v);
  v += dpp64<0x142, 0xA, false>(v);
  v += dpp64<0x143, 0xC, false>(v);
  return v;
}

__device__ inline uint64_t lane63_u64(uint64_t v) {
  const uint32_t lo = uint32_t(__builtin_amdgcn_readlane(int(uint32_t(v)), 63));
  const uint32_t hi = uint32_t(__builtin_amdgcn_readlane(int(uint32_t(v >> 32)), 63));
  return (uint64_t(hi) << 32) | lo;
}

// Wave totals, the same in every lane.  The FP64 one adds in the fixed order
// of the scan above, so equal inputs give equal sums.
__device__ inline double wave_sum(double v) {
  auto step = [](double x, uint64_t moved) { return x + __longlong_as_double(int64_t(moved)); };
  const auto bits = [](double x) { return uint64_t(__double_as_longlong(x)); };
  v = step(v, dpp64<0x111, 0xF, true>(bits(v)));
  v = step(v, dpp64<0x112, 0xF, true>(bits(v)));
  v = step(v, dpp64<0x114, 0xF, true>(bits(v)));
  v = step(v, dpp64<0x118, 0xF, true>(bits(v)));
  v = step(v, dpp64<0x142, 0xA, false>(bits(v)));
  v = step(v, dpp64<0x143, 0xC, false>(bits(v)));
  return __longlong_as_double(int64_t(lane63_u64(bits(v))));
}

__device__ inline uint64_t wave_sum_u64(uint64_t v) { return lane63_u64(wave_incl_scan_u64(v)); }

__device__ inline uint32_t wave_sum_u32(uint32_t v) {
  return uint32_t(__builtin_amdgcn_readlane(int(wave_incl_scan(v)), 63));
}

// ------------------------------------------------------------------ block hash
// Hash sender (CIERA page, section 3.1: per block a 128-bit hash of its
// exponents made of two independent 64-bit SplitMix64 hashes; a block is
// unchanged only when its hash equals the stored one).  A block's exponent
// fields, 8 at a time, form little-endian 64-bit words w_k; hash h is the sum
// mod 2^64, over the words that are not zero, of the SplitMix64 output
// function applied to w_k + s_h + (k + 1) g_h: the (k+1)-th output of a
// SplitMix64 generator (Steele, Lea and Flood, OOPSLA 2014) with seed
// w_k + s_h and increment g_h.  An all-zero block hashes to (0, 0), so a
// zeroed hash cache means all-zero previous exponents, as a zeroed exponent
// cache does, and the stream equals the exact-cache stream unless two
// different blocks' hashes collide.
constexpr uint64_t kHashSeed0 = 0ull, kHashGamma0 = 0x9E3779B97F4A7C15ull;
constexpr uint64_t kHashSeed1 = 0x243F6A8885A308D3ull, kHashGamma1 = 0xD1B54A32D192ED03ull;

__device__ inline uint64_t splitmix64_out(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__device__ inline uint64_t shfl_u64(uint64_t v, uint32_t src) {
  const uint32_t lo = uint32_t(__shfl(int(uint32_t(v)), int(src)));
  const uint32_t hi = uint32_t(__shfl(int(uint32_t(v >> 32)), int(src)));
  return (uint64_t(hi) << 32) | lo;
}

// ------------------------------------------------------------------ k_stats
// FP64 value of a BF16 pattern held in the top half of a float: BF16 -> FP32
// is exact (denormals are kept), FP32 -> FP64 is exact.
__device__ inline double widen_hi(uint32_t hi_bits) { return double(__uint_as_float(hi_bits)); }

// Partial sums of one unit's finite values (the checked path).
__device__ inline void stats_checked(const Unit& v, uint32_t cnt, double shift, double& s1, double& s2,
                                     uint32_t& nf) {
#pragma unroll
  for (uint32_t k = 0; k < 8u; k++) {
    const uint32_t b = (v.w[k >> 1] >> (16u * (k & 1u))) & 0xFFFFu;
    if (k < cnt && ((b >> 7) & 0xFFu) != 0xFFu) {
      const double d = widen_hi(b << 16) - shift;
      s1 += d;
      s2 = fma(d, d, s2);
      nf++;
    }
  }
}

// One unit's share of the variance sums, its values in order: no finiteness
// test for a full unit (a non-finite input makes the sums non-finite, and
// the thread then redoes its units with stats_checked).  k_stats and the
// speculative single-read write both add their units through this, so they
// produce the same bits.
__device__ inline void stats_unit(const Unit& v, uint32_t cnt, double shift, double& s1, double& s2, uint32_t& nf) {
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
}

// The shift of the variance sums: x[0], or 0 if x[0] is not finite.
__device__ inline double stats_shift(uint32_t first) {
  return (((first >> 7) & 0xFFu) != 0xFFu) ? widen_hi(first << 16) : 0.0;
}

// Word t of a chunk's bitmap (bit j set = block j changed) from the words its
// parts wrote (pw: kPartBitmapWords per part): part h keeps its own blocks'
// bits from bit 0 of its first word, or, when a block spans several parts,
// bit 0 = the part's share changed.
__device__ inline uint32_t chunk_bitmap_word(const uint32_t* pw, uint32_t t, uint32_t B) {
  if (32u * t >= kChunk / B) return 0u;  // past the chunk's last possible block
  if (B * 32u <= kPartValues) {  // 32 or more blocks per part
    const uint32_t nbp = kPartValues / B;
    return pw[kPartBitmapWords * ((32u * t) / nbp) + ((32u * t) % nbp) / 32u];
  }
  uint32_t w = 0;
  if (B <= kPartValues) {  // 1..16 blocks per part: chunk bits 0..63
    const uint32_t nbp = kPartValues / B;
    for (uint32_t h = 0; h < kParts; h++) {
      const uint32_t first = h * nbp;
      if (first / 32u == t) w |= (pw[kPartBitmapWords * h] & ((1u << nbp) - 1u)) << (first % 32u);
    }
  } else if (t == 0u) {
    const uint32_t ppb = B / kPartValues;
    for (uint32_t h = 0; h < kParts; h++) w |= (pw[kPartBitmapWords * h] & 1u) << (h / ppb);
  }
  return w;
}

// Workgroups are dealt round-robin over the chip's 8 XCDs, each with its own
// L2.  k_stats gives XCD x a contiguous range of parts, so that the small
// per-part records (partial sums, bitmap words) that share a 128-byte line
// are written from one L2.  The last (parts mod 8) workgroups keep their own
// index.
constexpr uint32_t kXcds = 8u;
__device__ inline uint32_t stats_part_of(uint32_t b, uint32_t parts) {
  const uint32_t per = parts / kXcds;
  if (b >= per * kXcds) return b;
  return (b % kXcds) * per + b / kXcds;
}

// One 256-thread workgroup per part (quarter chunk), units pu0 + 256 j + t;
// for self-planned tensors (kS = kSlices) one per slice of a part, units
// u0 + 256 j + t of the slice.  Per part (slice): FP64 variance partials; ciera: changed-block bits against the
// sender cache and the cache update; an exponent histogram of the values to
// code, and their count.  kHash: the sender cache is the block-hash cache
// (two u64 per block) instead of the exponents.
// kGiven: the fallback pass of a speculative encode (ws.spec), which returns
// at once if the speculation hit; else it takes each part's change bits from
// the records the speculative write left (no cache read, compare or write),
// and it clears only the planner slots' count words, keeping the variance
// sums k_sums wrote there.
template <bool kCiera, bool kHash, uint32_t kS, bool kGiven = false>
__global__ __launch_bounds__(kPartThreads) void k_stats(const uint16_t* __restrict__ x, uint64_t n,
                                                        uint8_t* __restrict__ cache, uint32_t log2B, Ws ws) {
  static_assert(kCiera || !kHash, "the hash sender is a ciera mode");
  static_assert(!kGiven || (!kHash && kS == 1u), "the speculative fallback is the exact sender's, one part each");
  if (kGiven && ws.ctrl->spec == kSpecHit) return;
  constexpr uint32_t kU = kUPT / kS;            // units per thread
  constexpr uint32_t kRange = kPartUnits / kS;  // units per workgroup
  // hash sender: first the part's exponent words (2048 u64), then the histogram
  __shared__ __attribute__((aligned(16))) uint32_t s_hist[kHistCopies * kBins];
  __shared__ uint32_t s_bits[kPartBitmapWords];
  __shared__ double s_s1[kPartWaves], s_s2[kPartWaves];
  __shared__ uint32_t s_nf[kPartWaves], s_wtot[kPartWaves];
  __shared__ uint64_t s_wh[2][kPartWaves];
  const uint32_t tid = threadIdx.x;
  const uint32_t lane = lane_id(), wave = tid >> 6;
  // the part (kS = 1) or slice this workgroup takes; its records sit at index wg
  const uint32_t wg = stats_part_of(blockIdx.x, gridDim.x);
  const uint64_t c = wg / (kParts * kS);
  const uint32_t h = (wg / kS) % kParts;
  const uint32_t slice = wg % kS;
  const uint64_t start = c * kChunk;
  const uint32_t nc = uint32_t(min(uint64_t(kChunk), n - start));
  const uint32_t nunits = (nc + 7u) / 8u;
  const uint32_t pu0 = h * kPartUnits;
  const uint32_t u0 = pu0 + slice * kRange;  // first unit of the workgroup
  const bool full = 8u * (u0 + kRange) <= nc;
  const uint32_t B = kCiera ? (1u << log2B) : 0u;
  const uint32_t blk0 = kCiera ? ((8u * pu0) >> log2B) : 0u;  // first block of the part
  if (!kHash)
    for (uint32_t i = tid; i < kHistCopies * kBins; i += kPartThreads) s_hist[i] = 0u;
  if (tid < kPartBitmapWords) s_bits[tid] = (kGiven && kCiera) ? ws.bitmap[uint64_t(wg) * kPartBitmapWords + tid] : 0u;
  if (ws.rstat && tid == 0 && h == 0u && slice == 0u) ws.rstat[c * kRstatStride] = 0u;  // rANS encode: the chunk's look-back word, not ready
  if (blockIdx.x == 0u) {
    // k_plan's slots: the count words not ready (words 3.. of each slot;
    // the fallback keeps words 0..2, the sums)
    uint64_t* sw = reinterpret_cast<uint64_t*>(ws.plan);
    for (uint32_t i = tid; i < kPlanMaxGroups * 8u; i += kPartThreads)
      if (!kGiven || (i & 7u) >= 3u) sw[i] = 0u;
    if (tid == 0) ws.ctrl->plan_fail = 0u;
  }
  // Hash sender, blocks within the part (a slice: within the slice): the hash
  // phase gives each block hb_threads consecutive threads (kU units each);
  // the last of them decides and fetches the block's stored hashes now.
  uint64_t* hcache = reinterpret_cast<uint64_t*>(cache);
  const uint32_t hb_threads = (kHash && B <= kPartValues) ? B / (8u * kU) : kPartThreads;
  const uint32_t sblk0 = kCiera ? ((8u * u0) >> log2B) - blk0 : 0u;  // the workgroup's first block in the part
  const uint64_t hblk = kHash ? c * (kChunk >> log2B) + blk0 + sblk0 + tid / hb_threads : 0u;  // global block
  const bool decider = kHash && B <= kPartValues && tid % hb_threads == hb_threads - 1u && (hblk << log2B) < n;
  uint64_t hc0 = 0, hc1 = 0;
  if (decider) {
    const uint4 e = *reinterpret_cast<const uint4*>(hcache + 2u * hblk);
    hc0 = (uint64_t(e.y) << 32) | e.x;
    hc1 = (uint64_t(e.w) << 32) | e.z;
  }

  // Load: all of a thread's 16-byte loads (and 8-byte cache loads) before use.
  Unit v[kU];
  uint2 old[kU];
  if (full) {
#pragma unroll
    for (uint32_t j = 0; j < kU; j++) v[j] = load_unit(x, start + 8ull * (u0 + j * kPartThreads + tid), 8u);
    if (kCiera && !kHash && !kGiven) {
#pragma unroll
      for (uint32_t j = 0; j < kU; j++)
        old[j] = *reinterpret_cast<const uint2*>(cache + start + 8ull * (u0 + j * kPartThreads + tid));
    }
  } else {
#pragma unroll
    for (uint32_t j = 0; j < kU; j++) {
      const uint32_t u = u0 + j * kPartThreads + tid;
      v[j].w[0] = v[j].w[1] = v[j].w[2] = v[j].w[3] = 0u;
      old[j] = make_uint2(0u, 0u);
      if (u < nunits) {
        v[j] = load_unit(x, start + 8ull * u, min(8u, nc - 8u * u));
        if (kCiera && !kHash && !kGiven) old[j] = load_bytes8(cache + start + 8ull * u, min(8u, nc - 8u * u));
      }
    }
  }
  // x[0] (the shift of the variance sums) and the given window byte, if any
  // (else x's first byte stands in): read after the part's loads are out,
  // both on every path, so that they share the part's round trip
  const uint32_t first = x[0];
  const uint32_t e0_byte = *(ws.e0_src ? ws.e0_src : reinterpret_cast<const uint8_t*>(x));
  const double shift = stats_shift(first);
  // a window base given in device memory that is out of range: the encode
  // writes nothing, so the sender cache is left as it was
  const bool keep_cache = ws.e0_src != nullptr && e0_byte > kMaxE0;
  __syncthreads();  // LDS cleared

  // Variance sums with no finite test per value: a non-finite input makes the
  // thread's sums non-finite (squares of finite BF16 values cannot overflow
  // FP64), and the thread then redoes its units on the checked path.  Ciera:
  // compare exponents with the cache and rewrite the bytes that differ; a
  // wave ballot gives the changed blocks among the wave's 64 units (lanes
  // [kL, kL + L) hold block k for L = B / 8 up to 64; from B = 512 on the 64
  // units lie in one block), set in s_bits by one atomic per wave.  Bit j of
  // `coded` says unit j's values are coded.
  double s1 = 0.0, s2 = 0.0;
  uint32_t nf = 0;
  uint32_t coded = kCiera ? 0u : 0xFFu;
  const uint32_t L = (B >= 512u) ? 64u : max(B / 8u, 8u);  // B >= 64 in ciera mode
  const uint64_t gmask = (L >= 64u) ? ~0ull : ((1ull << L) - 1u);
  // One copy of the unit loop for a part of 16384 values, one for a short
  // last part: the full copy carries no per-unit value counts.
  auto units = [&](auto full_c) {
    constexpr bool kF = decltype(full_c)::value;
#pragma unroll
    for (uint32_t j = 0; j < kU; j++) {
      const uint32_t u = u0 + j * kPartThreads + tid;
      bool diff = false, live = false;
      uint32_t ucnt = 0u;
      uint2 ue = make_uint2(0u, 0u);
      if (kF || u < nunits) {
        const uint32_t cnt = kF ? 8u : min(8u, nc - 8u * u);
        stats_unit(v[j], cnt, shift, s1, s2, nf);
        if (kCiera && !kGiven) {
          const uint2 e = unit_exponents(v[j]);
          const uint64_t keep = (cnt == 8u) ? ~0ull : ((1ull << (8u * (cnt & 7u))) - 1u);
          if (kHash) {
            reinterpret_cast<uint64_t*>(s_hist)[j * kPartThreads + tid] = ((uint64_t(e.y) << 32) | e.x) & keep;
          } else {
            diff = (((uint64_t(e.y ^ old[j].y) << 32) | (e.x ^ old[j].x)) & keep) != 0u;
            live = true;
            ucnt = cnt;
            ue = e;
          }
        }
      } else if (kHash) {
        reinterpret_cast<uint64_t*>(s_hist)[j * kPartThreads + tid] = 0u;  // past the data
      }
      if (kCiera && !kHash && !kGiven) {
        const uint64_t m = __ballot(diff);
        if (m != 0u) {
          if (live && !keep_cache && line_has_change(m)) store_bytes8(cache + start + 8ull * u, ucnt, ue);
          // first block of the wave's units, relative to the part
          const uint32_t lbw = ((8u * (u0 + j * kPartThreads + 64u * wave)) >> log2B) - blk0;
          uint32_t bits = 0;
          for (uint32_t k = 0; k < 64u / L; k++) bits |= ((m >> (k * L)) & gmask) ? (1u << k) : 0u;
          if (lane == 0u) atomicOr(&s_bits[lbw >> 5], bits << (lbw & 31u));
          if (B <= 512u) coded |= ((m >> (lane & ~(L - 1u))) & gmask) ? (1u << j) : 0u;
        }
      }
    }
  };
  if (full)
    units(std::true_type{});
  else
    units(std::false_type{});
  if (!(__builtin_isfinite(s1) && __builtin_isfinite(s2))) {
    s1 = 0.0;
    s2 = 0.0;
    nf = 0;
#pragma unroll
    for (uint32_t j = 0; j < kU; j++) {
      const uint32_t u = u0 + j * kPartThreads + tid;
      if (u < nunits) stats_checked(v[j], min(8u, nc - 8u * u), shift, s1, s2, nf);
    }
  }
  if (kHash) {
    // The range's exponent words are in LDS; thread t hashes units kU t ..
    // kU t + kU - 1 of the range (8 kU values), word k of its block being
    // unit k of it.
    static_assert(kU % 2u == 0u, "two words per 16-byte read");
    __syncthreads();
    const uint4* se = reinterpret_cast<const uint4*>(s_hist) + (kU / 2u) * tid;
    uint64_t w[kU];
#pragma unroll
    for (uint32_t i = 0; i < kU / 2u; i++) {
      const uint4 q = se[i];
      w[2u * i] = (uint64_t(q.y) << 32) | q.x;
      w[2u * i + 1u] = (uint64_t(q.w) << 32) | q.z;
    }
    const uint64_t k1 = uint64_t(((u0 + kU * tid) & ((B >> 3) - 1u)) + 1u);  // k + 1 of the first word
    uint64_t key0 = kHashSeed0 + k1 * kHashGamma0, key1 = kHashSeed1 + k1 * kHashGamma1;
    uint64_t p0 = 0, p1 = 0;
#pragma unroll
    for (uint32_t i = 0; i < kU; i++) {
      if (w[i]) {
        p0 += splitmix64_out(w[i] + key0);
        p1 += splitmix64_out(w[i] + key1);
      }
      key0 += kHashGamma0;
      key1 += kHashGamma1;
    }
    // The block's sum (mod 2^64) over its threads, in its last thread: a wave
    // scan minus the scan before the block's first lane, or, for blocks (or
    // a part's share of a block) wider than a wave, the waves' totals.
    uint64_t hs0 = p0, hs1 = p1;
    if (hb_threads > 1u) {
      const uint64_t i0 = wave_incl_scan_u64(p0), i1 = wave_incl_scan_u64(p1);
      if (hb_threads <= 64u) {
        const uint32_t lead = lane & ~(hb_threads - 1u);
        hs0 = i0 - shfl_u64(i0 - p0, lead);
        hs1 = i1 - shfl_u64(i1 - p1, lead);
      } else {
        if (lane == 63u) {
          s_wh[0][wave] = i0;
          s_wh[1][wave] = i1;
        }
        __syncthreads();
        const uint32_t wpb = hb_threads / 64u, wfirst = (wave / wpb) * wpb;
        hs0 = hs1 = 0u;
        for (uint32_t q = 0; q < wpb; q++) {
          hs0 += s_wh[0][wfirst + q];
          hs1 += s_wh[1][wfirst + q];
        }
      }
    }
    if (B <= kPartValues) {
      // decide: a changed block's new hashes go to the cache and its bit to s_bits
      bool changed = false;
      if (decider) {
        changed = hs0 != hc0 || hs1 != hc1;
        if (changed)
          *reinterpret_cast<uint4*>(hcache + 2u * hblk) =
              make_uint4(uint32_t(hs0), uint32_t(hs0 >> 32), uint32_t(hs1), uint32_t(hs1 >> 32));
      }
      if (hb_threads <= 64u) {
        const uint64_t m = __ballot(changed);  // set only at the blocks' last lanes
        if (m != 0u && lane == 0u) {
          const uint32_t per = 64u / hb_threads;  // blocks of this wave
          uint64_t bits = 0;
          for (uint32_t i = 0; i < per; i++) bits |= ((m >> (i * hb_threads + hb_threads - 1u)) & 1u) << i;
          const uint32_t b0 = sblk0 + wave * per;  // a multiple of per (sblk0 is one of 4 per)
          atomicOr(&s_bits[b0 >> 5], uint32_t(bits) << (b0 & 31u));
          if (per > 32u) atomicOr(&s_bits[(b0 >> 5) + 1u], uint32_t(bits >> 32));
        }
      } else if (changed) {
        const uint32_t b = sblk0 + tid / hb_threads;
        atomicOr(&s_bits[b >> 5], 1u << (b & 31u));
      }
    } else if (tid == kPartThreads - 1u) {
      // a block spans several parts: k_plan adds the parts' shares and decides
      ws.phash[2u * wg] = hs0;
      ws.phash[2u * wg + 1u] = hs1;
    }
    __syncthreads();  // the exponent words are no longer read; s_bits complete
    for (uint32_t i = tid; i < kHistCopies * kBins; i += kPartThreads) s_hist[i] = 0u;
    if (B > kPartValues) {
      coded = 0xFFu;
    } else {
#pragma unroll
      for (uint32_t j = 0; j < kU; j++) {
        const uint32_t lb = ((8u * (u0 + j * kPartThreads + tid)) >> log2B) - blk0;
        coded |= ((s_bits[lb >> 5] >> (lb & 31u)) & 1u) << j;
      }
    }
    __syncthreads();  // histogram cleared
  } else if (kCiera && kGiven) {
    // the part's recorded bits (in s_bits since before the first barrier)
    if (B > kPartValues) {
      coded = 0xFFu;
    } else {
#pragma unroll
      for (uint32_t j = 0; j < kU; j++) {
        const uint32_t lb = ((8u * (u0 + j * kPartThreads + tid)) >> log2B) - blk0;
        coded |= ((s_bits[lb >> 5] >> (lb & 31u)) & 1u) << j;
      }
    }
  } else if (kCiera && B > 512u) {
    // a block spans several waves: its bit is complete after the barrier.  A
    // part inside a block that spans several parts counts all of its values
    // (k_plan drops them if the block is unchanged).
    __syncthreads();
    if (B > kPartValues) {
      coded = 0xFFu;
    } else {
      const uint32_t w0 = s_bits[0];  // at most 16 blocks per part
#pragma unroll
      for (uint32_t j = 0; j < kU; j++) {
        const uint32_t lb = ((8u * (u0 + j * kPartThreads + 64u * wave)) >> log2B) - blk0;
        coded |= ((w0 >> lb) & 1u) << j;
      }
    }
  }

  // Exponent histogram of the coded values.  Word bin * kHistCopies + copy,
  // copy chosen by lane: equal exponents within a wave spread over
  // kHistCopies consecutive words (LDS banks).
  const uint32_t copy4 = 4u * (tid & (kHistCopies - 1u));
  if (full) {
    // every unit holds 8 values: the bin's byte offset comes straight from
    // the exponent bits of each half
    constexpr uint32_t kBinShift = 6u;  // log2(kHistCopies * 4)
    static_assert((1u << kBinShift) == kHistCopies * 4u, "kBinShift");
    constexpr uint32_t kBinMask = 0xFFu << kBinShift;
    uint8_t* hb = reinterpret_cast<uint8_t*>(s_hist);
#pragma unroll
    for (uint32_t j = 0; j < kU; j++) {
      if (!((coded >> j) & 1u)) continue;
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const uint32_t w = v[j].w[i];
        atomicAdd(reinterpret_cast<uint32_t*>(hb + (((w >> (7u - kBinShift)) & kBinMask) | copy4)), 1u);
        atomicAdd(reinterpret_cast<uint32_t*>(hb + (((w >> (23u - kBinShift)) & kBinMask) | copy4)), 1u);
      }
    }
  } else {
#pragma unroll
    for (uint32_t j = 0; j < kU; j++) {
      const uint32_t u = u0 + j * kPartThreads + tid;
      if (u >= nunits || !((coded >> j) & 1u)) continue;
      const uint32_t cnt = min(8u, nc - 8u * u);
      const uint2 e = unit_exponents(v[j]);
      uint32_t* hist = s_hist + copy4 / 4u;
#pragma unroll
      for (uint32_t k = 0; k < 8u; k++)
        if (k < cnt) atomicAdd(&hist[byte_of(e, k) * kHistCopies], 1u);
    }
  }
  s1 = wave_sum(s1);
  s2 = wave_sum(s2);
  nf = wave_sum_u32(nf);
  if (lane == 0u) {
    s_s1[wave] = s1;
    s_s2[wave] = s2;
    s_nf[wave] = nf;
  }
  __syncthreads();
  // One bin per thread: sum the copies and store the part's row (u16: a
  // part holds at most 16384 values); the bins add up to the coded count.
  {
    uint32_t sum = 0;
#pragma unroll
    for (uint32_t q = 0; q < kHistCopies; q++) sum += s_hist[tid * kHistCopies + ((q + tid) & (kHistCopies - 1u))];
    ws.hist[uint64_t(wg) * kBins + tid] = uint16_t(sum);
    sum = wave_sum_u32(sum);
    if (lane == 0u) s_wtot[wave] = sum;
  }
  if (kCiera && tid < kPartBitmapWords) ws.bitmap[uint64_t(wg) * kPartBitmapWords + tid] = s_bits[tid];
  __syncthreads();
  if (tid == 0) {
    double a = 0.0, b = 0.0;
    uint32_t m = 0, t = 0;
#pragma unroll
    for (uint32_t w = 0; w < kPartWaves; w++) {
      a += s_s1[w];
      b += s_s2[w];
      m += s_nf[w];
      t += s_wtot[w];
    }
    uint32_t nch = 0;
    if (kCiera) {
      if (B <= kPartValues) {
#pragma unroll
        for (uint32_t w = 0; w < kPartBitmapWords; w++) nch += __popc(s_bits[w]);
      } else {
        nch = s_bits[0] & 1u;
      }
    }
    Partial p;
    p.s1 = a;
    p.s2 = b;
    p.nf = m;
    p.nch = nch;
    p.coded = t;
    p.pad = 0u;
    ws.partial[wg] = p;
  }
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

// Chunk geometry shared by encode and decode: section offsets from the
// chunk's start, its value count and (ciera) changed-block count.
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

// Values passed between workgroups (k_plan's groups, the parts of the
// single-read encode) each sit in one word that also says whether it is
// there yet, so relaxed device-scope atomics suffice: no cache-wide
// acquire/release.  Every wait is bounded by Ws::spin_limit polls.
__device__ inline uint64_t load_relaxed(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline uint32_t load_relaxed(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void store_relaxed(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void store_relaxed(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Waits until ready() holds in every thread of the workgroup; false if the
// bound ran out first.
template <typename F>
__device__ inline bool wait_all(F ready, uint32_t limit) {
  for (uint32_t spins = 0;; spins++) {
    if (__syncthreads_and(ready())) return true;
    if (spins >= limit) return false;
    __builtin_amdgcn_s_sleep(1);
  }
}

__device__ inline uint64_t as_bits(double v) { return uint64_t(__double_as_longlong(v)); }
__device__ inline double from_bits(uint64_t v) { return __longlong_as_double((long long)v); }

// Sums of the workgroup's u64 values (all threads get the total; the order
// is fixed, which the FP64 variant below needs to give every group the same
// bits).
__device__ inline uint64_t plan_sum_u64(uint64_t v, uint64_t* s_w) {
  v = wave_sum_u64(v);
  __syncthreads();
  if (lane_id() == 0u) s_w[threadIdx.x >> 6] = v;
  __syncthreads();
  uint64_t t = 0;
#pragma unroll
  for (uint32_t w = 0; w < kPlanWaves; w++) t += s_w[w];
  return t;
}
__device__ inline double plan_sum_f64(double v, double* s_w) {
  v = wave_sum(v);
  __syncthreads();
  if (lane_id() == 0u) s_w[threadIdx.x >> 6] = v;
  __syncthreads();
  double t = 0.0;
#pragma unroll
  for (uint32_t w = 0; w < kPlanWaves; w++) t += s_w[w];
  return t;
}

// k_plan thread's chunk sizes over its rounds, kept in registers for ranges
// up to kRunRegs rounds (longer ones park them in the chunk table).
constexpr uint32_t kRunRegs = 8u;

// Coded values of one histogram row (a part's, or a slice's) with exponent
// in [E0, E0 + 6]: bins E0..E0+6 lie in the two 16-byte words q = E0 / 8 and
// q + 1 of the row (only in word q when E0 >= 248, and q + 1 is then past the
// row and not read), at u16 positions r .. r + 6, r = E0 mod 8.
// The coded values of a histogram row inside [E0, E0 + 6], from the row's 16
// counts starting at bin E0 & ~7: a = bins (E0 & ~7) + 0..7, b = the next 8
// (ignored past the row's end).
__device__ inline uint32_t window_count(uint4 a, uint4 b, uint32_t e0) {
  const uint32_t r0 = e0 & 7u;
  if ((e0 >> 3) == kBins / 8u - 1u) b = make_uint4(0u, 0u, 0u, 0u);
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  uint32_t sum = 0;
#pragma unroll
  for (uint32_t i = 0; i < 16u; i++) {
    const uint32_t cnt = (w[i >> 1] >> (16u * (i & 1u))) & 0xFFFFu;
    sum += (i - r0 < 7u) ? cnt : 0u;  // r0 <= i <= r0 + 6
  }
  return sum;
}

__device__ inline uint32_t row_in_window(const uint16_t* row_base, uint32_t e0) {
  const uint4* row = reinterpret_cast<const uint4*>(row_base) + (e0 >> 3);
  const uint4 b = (e0 >> 3) < kBins / 8u - 1u ? row[1] : make_uint4(0u, 0u, 0u, 0u);
  return window_count(row[0], b, e0);
}

// A chunk's layout from its parts' coded values, change fields (B <= 16384:
// the part's changed blocks; larger B: whether the part's share of its block
// changed) and coded values in the window: the escapes before each part
// (esc), the chunk's escapes and changed blocks, and its stream bytes.  A
// part's escapes are its coded values outside the window.  A part inside a
// block that spans several parts codes its values only if some part of the
// block saw a change.
__device__ inline uint64_t chunk_layout(uint32_t nc, uint32_t B, const uint32_t (&coded)[kParts],
                                        const uint32_t (&pnch)[kParts], const uint32_t (&inwin)[kParts],
                                        uint32_t (&esc)[kParts], uint32_t& esc_total, uint32_t& nch_out) {
  const uint32_t ppb = B > kPartValues ? B / kPartValues : 1u;  // parts per block when blocks span parts
  uint32_t nch = 0;
  if (B && B <= kPartValues) {
#pragma unroll
    for (uint32_t h = 0; h < kParts; h++) nch += pnch[h];
  } else if (B) {
    for (uint32_t first = 0; first < kParts; first += ppb) {
      uint32_t any = 0;
      for (uint32_t h = first; h < first + ppb; h++) any |= pnch[h];
      nch += any ? 1u : 0u;
    }
  }
  uint32_t acc = 0;
#pragma unroll
  for (uint32_t h = 0; h < kParts; h++) {
    bool codes = true;
    if (B > kPartValues) {
      uint32_t any = 0;
#pragma unroll
      for (uint32_t k = 0; k < kParts; k++) any |= (k / ppb == h / ppb) ? pnch[k] : 0u;
      codes = any != 0u;
    }
    esc[h] = acc;
    acc += codes ? coded[h] - inwin[h] : 0u;
  }
  esc_total = acc;
  nch_out = nch;
  const uint64_t planes = B ? uint64_t(nch) * B / 8u : cdiv(nc, 8u);
  return pad128(nc) + (B ? 128u : 0u) + 3u * pad128(planes) + pad128(acc);
}

// Chunk c's layout at window base e0 (one thread), from its parts' records
// in the workspace (one per part).  kHashBlocks: hash sender with blocks
// larger than a part, whose change decision k_stats leaves to the planner:
// the block's hashes are the sums of its parts' shares; a changed block's go
// to the hash cache, and each of its parts gets the block's flag (bit 0 of
// its bitmap word).
template <bool kHashBlocks>
__device__ inline uint64_t plan_chunk(uint64_t c, uint64_t n, uint32_t B, uint32_t e0, const Ws& ws,
                                      uint64_t* __restrict__ hcache, uint32_t (&esc)[kParts], uint32_t& esc_total,
                                      uint32_t& nch_out) {
  const uint32_t nc = uint32_t(min(uint64_t(kChunk), n - c * kChunk));
  const Partial* pp = ws.partial + c * kParts;
  uint32_t coded[kParts], pnch[kParts], inwin[kParts];
#pragma unroll
  for (uint32_t h = 0; h < kParts; h++) {
    coded[h] = pp[h].coded;
    pnch[h] = pp[h].nch;
    inwin[h] = row_in_window(ws.hist + (c * kParts + h) * kBins, e0);
  }
  if (kHashBlocks) {
    const uint32_t ppb = B / kPartValues;
    for (uint32_t q = 0; q < kChunk / B; q++) {
      const uint64_t blk = c * (kChunk / B) + q;
      bool changed = false;
      if (blk * B < n) {
        uint64_t s0 = 0, s1 = 0;
        for (uint32_t h = q * ppb; h < (q + 1u) * ppb; h++) {
          s0 += ws.phash[2u * (c * kParts + h)];
          s1 += ws.phash[2u * (c * kParts + h) + 1u];
        }
        const uint4 old = *reinterpret_cast<const uint4*>(hcache + 2u * blk);
        changed = s0 != ((uint64_t(old.y) << 32) | old.x) || s1 != ((uint64_t(old.w) << 32) | old.z);
        if (changed)
          *reinterpret_cast<uint4*>(hcache + 2u * blk) =
              make_uint4(uint32_t(s0), uint32_t(s0 >> 32), uint32_t(s1), uint32_t(s1 >> 32));
      }
      for (uint32_t h = q * ppb; h < (q + 1u) * ppb; h++) {
        pnch[h] = changed ? 1u : 0u;
        ws.bitmap[(c * kParts + h) * kPartBitmapWords] = changed ? 1u : 0u;
      }
    }
  }
  return chunk_layout(nc, B, coded, pnch, inwin, esc, esc_total, nch_out);
}

// The window base from the G planner groups' variance sums (k_sums wrote
// them), added in group order: every thread of every caller gets the same
// bits, and so the same window base.
__device__ inline uint32_t plan_e0(const PlanSlot* slot, uint32_t G, double* s_f, uint64_t* s_u) {
  const uint32_t tid = threadIdx.x;
  double ga = 0.0, gb = 0.0;
  uint64_t gm = 0;
  if (tid < G) {
    ga = from_bits(slot[tid].s1);
    gb = from_bits(slot[tid].s2);
    gm = slot[tid].nf;
  }
  const double s1 = plan_sum_f64(ga, s_f);
  const double s2 = plan_sum_f64(gb, s_f);
  const uint64_t nf = plan_sum_u64(gm, s_u);
  double var = 0.0;
  if (nf >= 2u) {
    var = (s2 - s1 * s1 / double(nf)) / double(nf - 1u);
    if (!(var > 0.0)) var = 0.0;
  }
  return window_base(var, nf);
}

// The planner's groups: group g of G takes chunks [g per, (g + 1) per).
// k_sums: each group adds up its parts' variance partials in a fixed order
// and stores them in its slot.  Nothing waits; k_plan, the next launch,
// reads every slot.
__global__ __launch_bounds__(kPlanThreads) void k_sums(uint64_t nchunks, uint64_t per, Ws ws) {
  __shared__ double s_f[kPlanWaves];
  __shared__ uint64_t s_u[kPlanWaves];
  const uint32_t tid = threadIdx.x, g = blockIdx.x;
  const uint64_t c0 = min(nchunks, per * g), c1 = min(nchunks, c0 + per);
  double a = 0.0, b = 0.0;
  uint64_t m = 0;
  for (uint64_t i = kParts * c0 + tid; i < kParts * c1; i += kPlanThreads) {
    const Partial& p = ws.partial[i];
    a += p.s1;
    b += p.s2;
    m += p.nf;
  }
  a = plan_sum_f64(a, s_f);
  b = plan_sum_f64(b, s_f);
  m = plan_sum_u64(m, s_u);
  if (tid == 0) {
    ws.plan[g].s1 = as_bits(a);
    ws.plan[g].s2 = as_bits(b);
    ws.plan[g].nf = m;
  }
}

// Speculative encode: the window base from the variance, by k_plan's own
// first step, against the hinted one the single-read write used (ctrl->e0).
// One workgroup; ctrl->spec = kSpecHit when they agree and every write
// workgroup finished, so that the fallback launches (k_stats with the
// recorded change bits, k_plan, k_write) return at once.
__global__ __launch_bounds__(kPlanThreads) void k_check(uint32_t G, Ws ws) {
  __shared__ double s_f[kPlanWaves];
  __shared__ uint64_t s_u[kPlanWaves];
  const uint32_t e0 = plan_e0(ws.plan, G, s_f, s_u);
  if (threadIdx.x == 0)
    ws.ctrl->spec = (ws.ctrl->spec_fail == 0u && ws.ctrl->e0 == e0) ? kSpecHit : 0u;
}

// k_plan, the same groups: (1) every group adds the G groups' sums in group
// order, so all pick the same E0.  (2) Each group sizes its chunks: a
// part's escapes are its coded values minus those with exponent in
// [E0, E0 + 6], read off its histogram row, so each chunk's size is exact
// (the size exchange of the digest's Figure 1, done on one GPU).  A group
// publishes its bytes, escapes and changed blocks and adds up those of the
// groups before it for its base offset; the last group also has the totals.
// Group 0 writes the header's fixed fields, the last group the totals and
// *out_size.  A group waits only on lower-numbered groups, which the GPU
// dispatches first, so the waits end whatever else runs on the GPU; if one
// does not end in its bound, the group sets ctrl->plan_fail and k_write
// writes nothing.  kHashBlocks: hash sender with blocks larger than a part,
// whose change decision k_stats leaves to this kernel (hcache is then the
// hash cache).
template <bool kHashBlocks>
__global__ __launch_bounds__(kPlanThreads) void k_plan(uint64_t n, uint64_t nchunks, uint64_t per, uint32_t B,
                                                       int e0_override, uint8_t* __restrict__ out,
                                                       uint64_t* __restrict__ out_size, uint64_t* __restrict__ hcache,
                                                       Ws ws) {
  __shared__ double s_f[kPlanWaves];
  __shared__ uint64_t s_u[kPlanWaves];
  __shared__ uint32_t s_e0;
  const uint32_t tid = threadIdx.x;
  const uint32_t g = blockIdx.x, G = gridDim.x;
  const uint64_t c0 = min(nchunks, per * g), c1 = min(nchunks, c0 + per);
  uint64_t* hd = reinterpret_cast<uint64_t*>(out);
  uint64_t* table = reinterpret_cast<uint64_t*>(out + kHeader);
  const uint64_t base = table_end(nchunks);
  // a speculative encode whose hinted window was right: nothing to plan
  if (ws.spec && ws.ctrl->spec == kSpecHit) return;
  PlanSlot* slot = ws.plan;
  if (g == 0u) {
    if (tid == 0) ws.ctrl->n_err_slots = nchunks * kParts;
    // the padding words after the chunk table and the escape index
    for (uint64_t i = 2u * nchunks + 1u + tid; i < (base - kHeader) / 8u; i += kPlanThreads) table[i] = 0u;
  }

  // (1) the variance from every group's sums (k_sums wrote them)
  const uint32_t e0_sigma = plan_e0(slot, G, s_f, s_u);
  if (tid == 0) {
    const uint32_t e0 = (e0_override >= 0) ? uint32_t(e0_override) : e0_sigma;
    s_e0 = e0;
    if (g == 0u) {
      ws.ctrl->e0 = e0;
      const uint32_t magic = B ? 0x52454943u /* "CIER" */ : 0x3350495Au /* "ZIP3" */;
      hd[0] = uint64_t(magic) | (1ull << 32) | (uint64_t(B ? 1u : 0u) << 48) | (uint64_t(e0) << 56);
      hd[1] = n;
      hd[2] = uint64_t(B) | (uint64_t(kChunk) << 32);
      hd[3] = nchunks;
      for (int i = 7; i < 16; i++) hd[i] = 0u;
    }
  }
  __syncthreads();
  const uint32_t e0 = s_e0;

  // (2) sizes of the group's chunks, one per thread per round of 256.
  auto chunk_size = [&](uint64_t c, uint64_t& esc_out, uint64_t& nch_out) -> uint64_t {
    uint32_t esc[kParts], acc, nch;
    const uint64_t size = plan_chunk<kHashBlocks>(c, n, B, e0, ws, hcache, esc, acc, nch);
#pragma unroll
    for (uint32_t h = 0; h < kParts; h++) ws.partesc[c * kParts + h] = esc[h];
    ws.chunkesc[c] = acc;
    table[nchunks + 1u + c] = uint64_t(esc[0]) | (uint64_t(esc[1]) << 16) | (uint64_t(esc[2]) << 32) |
                              (uint64_t(esc[3]) << 48);
    esc_out += acc;
    nch_out += nch;
    return size;
  };
  // one round: the chunk's offset from the group's start; carry = the
  // group's bytes so far
  uint64_t carry = 0, g_esc = 0, g_nch = 0;
  auto round = [&](uint64_t r) -> uint64_t {
    const uint64_t c = c0 + r * kPlanThreads + tid;
    const uint64_t size = (c < c1) ? chunk_size(c, g_esc, g_nch) : 0u;
    const uint64_t incl = wave_incl_scan_u64(size);
    __syncthreads();
    if (lane_id() == 63u) s_u[tid >> 6] = incl;
    __syncthreads();
    uint64_t before = carry + incl - size, total = 0;
#pragma unroll
    for (uint32_t w = 0; w < kPlanWaves; w++) {
      before += (w < (tid >> 6)) ? s_u[w] : 0u;
      total += s_u[w];
    }
    carry += total;
    return before;
  };
  const uint64_t rounds = cdiv(c1 - c0, kPlanThreads);
  uint64_t local[kRunRegs];
  if (rounds <= kRunRegs) {
#pragma unroll
    for (uint32_t r = 0; r < kRunRegs; r++) local[r] = (r < rounds) ? round(r) : 0u;
  } else {
    for (uint64_t r = 0; r < rounds; r++) {
      const uint64_t before = round(r);
      const uint64_t c = c0 + r * kPlanThreads + tid;
      if (c < c1) table[c] = before;
    }
  }
  const uint64_t own_bytes = carry;
  const uint64_t own_esc = plan_sum_u64(g_esc, s_u);
  const uint64_t own_nch = plan_sum_u64(g_nch, s_u);
  if (tid == 0) {
    store_relaxed(&slot[g].bytes, kSlotReady | own_bytes);
    store_relaxed(&slot[g].esc, kSlotReady | own_esc);
    store_relaxed(&slot[g].nch, kSlotReady | own_nch);
  }
  // the groups before this one
  uint64_t pb = 0, pe = 0, pn = 0;
  const bool preds_in = wait_all(
      [&] {
        if (tid >= g) return true;
        const uint64_t w1 = load_relaxed(&slot[tid].bytes), w2 = load_relaxed(&slot[tid].esc);
        const uint64_t w3 = load_relaxed(&slot[tid].nch);
        pb = w1 & ~kSlotReady;
        pe = w2 & ~kSlotReady;
        pn = w3 & ~kSlotReady;
        return (w1 & w2 & w3 & kSlotReady) != 0u;
      },
      ws.spin_limit);
  if (!preds_in) {
    if (tid == 0) store_relaxed(&ws.ctrl->plan_fail, 1u);
    return;
  }
  if (tid >= g) pb = pe = pn = 0u;
  const uint64_t at = base + plan_sum_u64(pb, s_u);
  const uint64_t esc_before = plan_sum_u64(pe, s_u);
  const uint64_t nch_before = plan_sum_u64(pn, s_u);
  if (rounds <= kRunRegs) {
#pragma unroll
    for (uint32_t r = 0; r < kRunRegs; r++) {
      const uint64_t c = c0 + uint64_t(r) * kPlanThreads + tid;
      if (r < rounds && c < c1) table[c] = at + local[r];
    }
  } else {
    for (uint64_t c = c0 + tid; c < c1; c += kPlanThreads) table[c] += at;
  }
  if (g + 1u == G && tid == 0) {
    const uint64_t total = at + own_bytes;
    table[nchunks] = total;
    hd[4] = total;
    hd[5] = nch_before + own_nch;
    hd[6] = esc_before + own_esc;
    *out_size = total;
  }
}

// ------------------------------------------------------------------ k_write
__device__ inline void zero_fill(uint8_t* __restrict__ p, uint64_t from, uint64_t to, uint32_t nthreads) {
  for (uint64_t i = from + threadIdx.x; i < to; i += nthreads) p[i] = 0u;
}

// Block-wide (256 threads) sum and inclusive scan of u32 values.
__device__ inline uint32_t part_sum_u32(uint32_t v, uint32_t* s_w) {
  v = wave_sum_u32(v);
  __syncthreads();
  if (lane_id() == 0u) s_w[threadIdx.x >> 6] = v;
  __syncthreads();
  uint32_t t = 0;
#pragma unroll
  for (uint32_t w = 0; w < kPartWaves; w++) t += s_w[w];
  return t;
}
__device__ inline uint32_t part_incl_scan_u32(uint32_t v, uint32_t* s_w) {
  const uint32_t incl = wave_incl_scan(v);
  __syncthreads();
  if (lane_id() == 63u) s_w[threadIdx.x >> 6] = incl;
  __syncthreads();
  uint32_t before = 0;
#pragma unroll
  for (uint32_t w = 0; w < kPartWaves; w++) before += (w < (threadIdx.x >> 6)) ? s_w[w] : 0u;
  return before + incl;
}

// Escape positions within a part: cnt[j] (0..8) per unit, units ordered
// (j, wave, lane).  base[j] receives the escapes in earlier units of the part;
// returns the part's total.  Every thread of the workgroup must call it.
// kSettle: base[] is computed before the first barrier, so the scan's partial
// sums die there; otherwise the compiler may keep them (a dozen registers)
// until the totals come back, which measured faster for k_write alone.
template <uint32_t N, bool kSettle = true>
__device__ inline uint32_t part_escape_scan(const uint32_t (&cnt)[N], uint32_t (&base)[N],
                                            uint32_t* s_tot /* N * kPartWaves + 1 */) {
  static_assert(N % 2u == 0u && N <= kUPT, "unit pairs, at most kUPT per thread");
  const uint32_t lane = lane_id();
  const uint32_t wave = threadIdx.x >> 6;
  // two counts per 32-bit word (16-bit fields; a wave's sum is at most 512)
#pragma unroll
  for (uint32_t p = 0; p < N / 2u; p++) {
    const uint32_t packed = cnt[2 * p] | (cnt[2 * p + 1] << 16);
    const uint32_t incl = wave_incl_scan(packed);
    uint32_t excl = incl - packed;
    if (kSettle) __asm__ volatile("" : "+v"(excl));  // opaque: the partial sums end here
    base[2 * p] = excl & 0xFFFFu;
    base[2 * p + 1] = excl >> 16;
    if (lane == 63u) {
      s_tot[(2 * p) * kPartWaves + wave] = incl & 0xFFFFu;
      s_tot[(2 * p + 1) * kPartWaves + wave] = incl >> 16;
    }
  }
  __syncthreads();
  constexpr uint32_t kEntries = N * kPartWaves;
  if (wave == 0) {
    const uint32_t a = (lane < kEntries) ? s_tot[lane] : 0u;
    const uint32_t incl = wave_incl_scan(a);
    if (lane < kEntries) s_tot[lane] = incl - a;
    if (lane == 63u) s_tot[kEntries] = incl;
  }
  __syncthreads();
#pragma unroll
  for (uint32_t j = 0; j < N; j++) base[j] += s_tot[j * kPartWaves + wave];
  return s_tot[kEntries];
}

// Plane bytes (one per coded unit slot) before unit u of a ciera chunk: the
// slots of all changed blocks before u's block, plus u's offset in its block
// if that block is changed.  Units past the chunk's last block see all slots.
__device__ inline uint32_t coded_before(uint32_t u, const uint32_t* s_bits, const uint32_t* s_rank, uint32_t log2B,
                                        uint32_t nb, uint32_t nch) {
  const uint32_t upb_log = log2B - 3u;  // units per block = B / 8
  const uint32_t blk = u >> upb_log;
  if (blk >= nb) return nch << upb_log;
  const uint32_t word = s_bits[blk >> 5];
  const uint32_t rank = s_rank[blk >> 5] + __popc(word & ((1u << (blk & 31u)) - 1u));
  const bool changed = (word >> (blk & 31u)) & 1u;
  return (rank << upb_log) + (changed ? (u & ((1u << upb_log) - 1u)) : 0u);
}

// Bitmap words into LDS with the changed-block counts before each word;
// wave 0 only.
__device__ inline void stage_bitmap(uint32_t w, uint32_t* s_bits, uint32_t* s_rank) {
  const uint32_t tid = threadIdx.x;
  const uint32_t pc = __popc(w);
  const uint32_t incl = wave_incl_scan(pc);
  if (tid < kBitmapWords) {
    s_bits[tid] = w;
    s_rank[tid] = incl - pc;
  }
}

// One part of a chunk.  Its stream offset, the escapes before it in its chunk
// and the chunk's escape total all come from k_plan, so the part waits on
// nothing: load, code, write.
// Tensors of at most kSelfPlanChunks chunks are planned by one group; the
// write kernel then plans for itself instead (two launches fewer for a
// shard-sized tensor): every workgroup adds the variance sums of k_stats'
// records in the one-group planner's order, sizes every chunk and scans the
// sizes in one wave.  With one record per part that gives the planner's bits
// and window base; with one per slice (ws.ss > 1) the sums round in another
// order, which can move the window base only where the variance lies within
// that rounding of a threshold.  Workgroup 0 writes the header and totals,
// the first slice of part 0 of each chunk its table and escape-index entries.
constexpr uint64_t kSelfPlanChunks = kPlanMinChunks;
static_assert(kSelfPlanChunks <= 64u, "one wave scans every chunk");
struct SelfPlan {
  uint64_t begin;
  uint32_t e0, esc_before, esc_chunk, esc_part;
  // one record per slice (ws.ss > 1): the escapes of slice `slice` of the
  // part and those of the part's slices before it
  uint32_t esc_slice, esc_slice_before;
};
// The self-plan in two steps, so that the workgroup codes its values while
// the histogram windows are on their way.  Step one: the window base from the
// statistics records (thread t adds record t), then the loads of each
// record's histogram counts around the window, issued and not waited for.
// Both loads are taken on every path (record 0 stands in for threads past
// the records, the row's last 16 bytes for the 16 past its end), so that no
// later load waits for them.
struct PlanStart {
  uint32_t e0;  // kBadE0: the given window base is out of range
  uint32_t r_coded, r_nch;
  uint4 wa, wb;
};
__device__ inline PlanStart self_plan_start(uint64_t nchunks, uint32_t wg, int e0_override,
                                            uint8_t* __restrict__ out, uint64_t* __restrict__ out_size,
                                            const Ws& ws) {
  __shared__ double s_f[kPlanWaves];
  __shared__ uint64_t s_u[kPlanWaves];
  __shared__ uint32_t s_e0;
  static_assert(kPartThreads == kPlanThreads, "the planner's reduction order");
  static_assert(kSelfPlanChunks * kParts * kSlices <= kPlanThreads, "one record per thread");
  const uint32_t tid = threadIdx.x;
  const uint32_t nrec = uint32_t(kParts * nchunks) * ws.ss;
  // a window base given in device memory, read with the records
  const uint32_t e0_given = ws.e0_src ? uint32_t(ws.e0_src[0]) : 0u;
  // Thread t takes record t, as the one-group planner's k_sums takes part t.
  // The load is taken on every path (the last record stands in past the
  // records and adds nothing), so it goes out with the loads before it.
  const Partial p = ws.partial[min(tid, nrec - 1u)];
  const bool own = tid < nrec;
  double a = own ? p.s1 : 0.0, b = own ? p.s2 : 0.0;
  uint64_t m = own ? p.nf : 0u;
  PlanStart r;
  r.r_coded = own ? p.coded : 0u;
  r.r_nch = own ? p.nch : 0u;
  a = plan_sum_f64(a, s_f);
  b = plan_sum_f64(b, s_f);
  m = plan_sum_u64(m, s_u);
  if (tid == 0) {
    double var = 0.0;
    if (m >= 2u) {
      var = (b - a * a / double(m)) / double(m - 1u);
      if (!(var > 0.0)) var = 0.0;
    }
    s_e0 = ws.e0_src ? e0_given : ((e0_override >= 0) ? uint32_t(e0_override) : window_base(var, m));
  }
  __syncthreads();
  const uint32_t e0 = s_e0;
  r.e0 = e0;
  if (e0 > kMaxE0) {
    // only from device memory: the stream gets its first header word alone,
    // whose E0 byte keeps the bad value (a decoder refuses it, and so does a
    // next encode taking its window base from that byte), and no size
    if (wg == 0u && tid == 0u) {
      *reinterpret_cast<uint64_t*>(out) = uint64_t(e0) << 56;
      *out_size = 0u;
      ws.ctrl->e0 = kBadE0;
      ws.ctrl->n_err_slots = gridDim.x;
    }
    r.e0 = kBadE0;
    return r;
  }
  const uint4* row = reinterpret_cast<const uint4*>(ws.hist + uint64_t(tid < nrec ? tid : 0u) * kBins) + (e0 >> 3);
  r.wa = row[0];
  r.wb = row[(e0 >> 3) < kBins / 8u - 1u ? 1 : 0];
  return r;
}

// Step two: each record's coded values in the window, the chunks' layout and
// offsets, the chunk table, the header; the workgroup's part and slice
// entries.
__device__ inline SelfPlan self_plan_finish(uint64_t n, uint64_t nchunks, uint64_t c, uint32_t h, uint32_t slice,
                                            bool lead, uint32_t wg, uint32_t B, const PlanStart& ps,
                                            uint8_t* __restrict__ out, uint64_t* __restrict__ out_size,
                                            const Ws& ws) {
  __shared__ uint64_t s_r[5];
  __shared__ uint32_t s_pc[kSelfPlanChunks * kParts], s_pn[kSelfPlanChunks * kParts], s_pi[kSelfPlanChunks * kParts];
  __shared__ uint32_t s_re[kPlanThreads];  // each record's escapes
  const uint32_t tid = threadIdx.x;
  const uint32_t ss = ws.ss;
  const uint32_t nrec = uint32_t(kParts * nchunks) * ss;
  const uint32_t e0 = ps.e0;
  uint32_t r_coded = ps.r_coded, r_nch = ps.r_nch;
  // Each record's coded values in the window; a part's records (ss
  // consecutive lanes of one wave) added by lane exchanges; then one thread
  // per chunk lays the chunk out.
  uint32_t r_in = tid < nrec ? window_count(ps.wa, ps.wb, e0) : 0u;
  // a record's escapes (used with one record per slice, where no block spans
  // slices, so that all of a record's coded values are written)
  s_re[tid] = r_coded - r_in;
  for (uint32_t off = 1u; off < ss; off <<= 1) {
    r_coded += uint32_t(__shfl_xor(int(r_coded), int(off)));
    r_nch += uint32_t(__shfl_xor(int(r_nch), int(off)));
    r_in += uint32_t(__shfl_xor(int(r_in), int(off)));
  }
  if (tid < nrec && tid % ss == 0u) {
    s_pc[tid / ss] = r_coded;
    s_pn[tid / ss] = r_nch;
    s_pi[tid / ss] = r_in;
  }
  __syncthreads();
  uint32_t esc[kParts] = {0u, 0u, 0u, 0u}, esc_total = 0u, nch = 0u;
  uint64_t size = 0;
  if (tid < nchunks) {
    uint32_t coded[kParts], pnch[kParts], inwin[kParts];
#pragma unroll
    for (uint32_t q = 0; q < kParts; q++) {
      coded[q] = s_pc[kParts * tid + q];
      pnch[q] = s_pn[kParts * tid + q];
      inwin[q] = s_pi[kParts * tid + q];
    }
    const uint32_t nc = uint32_t(min(uint64_t(kChunk), n - uint64_t(tid) * kChunk));
    size = chunk_layout(nc, B, coded, pnch, inwin, esc, esc_total, nch);
  }
  const uint64_t base = table_end(nchunks);
  uint64_t* hd = reinterpret_cast<uint64_t*>(out);
  uint64_t* table = reinterpret_cast<uint64_t*>(out + kHeader);
  if (tid < 64u) {
    const uint64_t incl = wave_incl_scan_u64(size);
    if (tid == c) {
      uint32_t eb = 0u, en = esc_total;  // part h's entry and the next part's (constant indices)
#pragma unroll
      for (uint32_t q = 0; q < kParts; q++) {
        eb = (q == h) ? esc[q] : eb;
        en = (q == h + 1u) ? esc[q] : en;
      }
      s_r[0] = base + incl - size;
      s_r[2] = eb;
      s_r[3] = esc_total | (uint64_t(en - eb) << 32);
      if (lead) {
        table[c] = base + incl - size;
        table[nchunks + 1u + c] = uint64_t(esc[0]) | (uint64_t(esc[1]) << 16) | (uint64_t(esc[2]) << 32) |
                                  (uint64_t(esc[3]) << 48);
      }
    }
    if (wg == 0u) {
      const uint64_t t_esc = wave_sum_u64(esc_total), t_nch = wave_sum_u64(nch);
      if (tid + 1u == nchunks) {
        table[nchunks] = base + incl;
        hd[4] = base + incl;
        *out_size = base + incl;
      }
      if (tid == 0u) {
        const uint32_t magic = B ? 0x52454943u /* "CIER" */ : 0x3350495Au /* "ZIP3" */;
        hd[0] = uint64_t(magic) | (1ull << 32) | (uint64_t(B ? 1u : 0u) << 48) | (uint64_t(e0) << 56);
        hd[1] = n;
        hd[2] = uint64_t(B) | (uint64_t(kChunk) << 32);
        hd[3] = nchunks;
        hd[5] = t_nch;
        hd[6] = t_esc;
        for (int i = 7; i < 16; i++) hd[i] = 0u;
        ws.ctrl->e0 = e0;
        ws.ctrl->n_err_slots = gridDim.x;
      }
    }
  }
  if (wg == 0u)  // the padding words after the chunk table and the escape index
    for (uint64_t i = 2u * nchunks + 1u + tid; i < (base - kHeader) / 8u; i += kPartThreads) table[i] = 0u;
  if (tid == 0u) {
    const uint32_t rec0 = uint32_t(c * kParts + h) * ss;
    uint32_t before = 0u;
    for (uint32_t q = 0; q < slice && q < ss; q++) before += s_re[rec0 + q];
    s_r[4] = (uint64_t(slice < ss ? s_re[rec0 + slice] : 0u) << 32) | before;
  }
  __syncthreads();
  SelfPlan r;
  r.begin = s_r[0];
  r.e0 = e0;
  r.esc_before = uint32_t(s_r[2]);
  r.esc_chunk = uint32_t(s_r[3]);
  r.esc_part = uint32_t(s_r[3] >> 32);
  r.esc_slice_before = uint32_t(s_r[4]);
  r.esc_slice = uint32_t(s_r[4] >> 32);
  return r;
}

// A thread's escapes (the raw exponent bytes of its units' code-0 values) to
// the part's LDS staging at their ranks base[j], in value order.
template <uint32_t N>
__device__ inline void stage_escapes(const Unit (&v)[N], const uint32_t (&emask)[N], const uint32_t (&base)[N],
                                     uint8_t* s_esc) {
#pragma unroll
  for (uint32_t j = 0; j < N; j++) {
    uint32_t em = emask[j];
    if (em) {
      const uint2 e = unit_exponents(v[j]);
      uint32_t at = base[j];
      while (em) {
        const uint32_t k = __builtin_ctz(em);
        em &= em - 1u;
        s_esc[at++] = uint8_t(byte_of(e, k));
      }
    }
  }
}

// The same from the units' exponent bytes, with the escape masks packed four
// to a word (unit j's in byte j % 4 of em4[j / 4]).
template <uint32_t N>
__device__ inline void stage_escapes_ex(const uint2 (&ex)[N], const uint32_t (&em4)[N / 4u], const uint32_t (&base)[N],
                                        uint8_t* s_esc) {
#pragma unroll
  for (uint32_t j = 0; j < N; j++) {
    uint32_t em = (em4[j / 4u] >> (8u * (j % 4u))) & 0xFFu;
    uint32_t at = base[j];
    while (em) {
      const uint32_t k = __builtin_ctz(em);
      em &= em - 1u;
      s_esc[at++] = uint8_t(byte_of(ex[j], k));
    }
  }
}

// One part of a chunk (kS = 1) or one of its kS slices (self-planned
// tensors only): a slice codes units [u0, u0 + kPartUnits / kS) and counts
// the escapes of the part's units before u0 to place its own.
template <bool kCiera, bool kSelfPlan, uint32_t kS>
__global__ __launch_bounds__(kPartThreads) void k_write(const uint16_t* __restrict__ x, uint64_t n,
                                                        uint32_t log2B, uint8_t* __restrict__ out,
                                                        uint64_t capacity, uint64_t* __restrict__ out_size,
                                                        int e0_override, Ws ws) {
  static_assert(kS == 1u || kSelfPlan, "slices only for self-planned tensors");
  constexpr uint32_t kU = kUPT / kS;             // units per thread
  constexpr uint32_t kRange = kPartUnits / kS;   // units per workgroup
  constexpr uint32_t kEarly = kUPT - kU;         // most units per thread before u0
  __shared__ __attribute__((aligned(16))) uint8_t s_planes[3u * kStage];
  __shared__ __attribute__((aligned(16))) uint8_t s_esc[kPartEscStage];
  __shared__ uint32_t s_bits[kBitmapWords];
  __shared__ uint32_t s_rank[kBitmapWords];
  __shared__ uint32_t s_tot[kUPT * kPartWaves + 1];
  __shared__ uint32_t s_zw[kPartWaves];
  const uint32_t tid = threadIdx.x;
  const uint32_t wg = blockIdx.x;
  const uint32_t c = wg / (kParts * kS);
  const uint32_t h = (wg / kS) % kParts;
  const uint32_t slice = wg % kS;
  const bool last_part = h + 1u == kParts;
  const bool final_slice = slice + 1u == kS;
  const uint32_t B = 1u << log2B;
  if (ws.spec && ws.ctrl->spec == kSpecHit) return;  // a speculative encode that hit: the stream is written
  const uint64_t start = uint64_t(c) * kChunk;
  const uint32_t nc = uint32_t(min(uint64_t(kChunk), n - start));
  const uint32_t nunits = (nc + 7u) / 8u;
  const uint32_t pu0 = h * kPartUnits;
  const uint32_t u0 = pu0 + slice * kRange;

  // Load the range first: all of a thread's 16-byte loads go out before any
  // is used.  A slice whose escapes the plan does not count per slice (the
  // statistics kept one record per part) also loads the part's units before
  // it, to count their escapes.
  const bool counted = kS > 1u && ws.ss == kS;  // the plan has this slice's escapes
  Unit v[kU];
  if (8u * (u0 + kRange) <= nc) {
#pragma unroll
    for (uint32_t j = 0; j < kU; j++) v[j] = load_unit(x, start + 8ull * (u0 + j * kPartThreads + tid), 8u);
  } else {
#pragma unroll
    for (uint32_t j = 0; j < kU; j++) {
      const uint32_t u = u0 + j * kPartThreads + tid;
      v[j].w[0] = v[j].w[1] = v[j].w[2] = v[j].w[3] = 0u;
      if (u < nunits) v[j] = load_unit(x, start + 8ull * u, min(8u, nc - 8u * u));
    }
  }
  // (thread t's units before u0 are pu0 + 256 k + t, k < slice * kU; all
  // hold 8 values unless the data ends before u0)
  Unit ve[kEarly > 0u ? kEarly : 1u];
#pragma unroll
  for (uint32_t k = 0; k < kEarly; k++) ve[k].w[0] = ve[k].w[1] = ve[k].w[2] = ve[k].w[3] = 0u;
  if (kEarly > 0u && !counted) {
    const uint32_t nearly = slice * kU;
    if (8u * u0 <= nc) {
#pragma unroll
      for (uint32_t k = 0; k < kEarly; k++)
        if (k < nearly) ve[k] = load_unit(x, start + 8ull * (pu0 + k * kPartThreads + tid), 8u);
    } else {
#pragma unroll
      for (uint32_t k = 0; k < kEarly; k++) {
        const uint32_t u = pu0 + k * kPartThreads + tid;
        if (k < nearly && u < nunits) ve[k] = load_unit(x, start + 8ull * u, min(8u, nc - 8u * u));
      }
    }
  }
  const uint64_t nchunks = cdiv(n, kChunk);
  uint64_t begin = 0;
  uint32_t esc_before = 0u, esc_chunk = 0u, esc_part = 0u, e0;
  uint32_t esc_slice = 0u, esc_slice_before = 0u;
  // self-planned: the chunk's bitmap words are fetched with the plan's inputs
  __shared__ uint32_t s_pw[kSelfPlan ? kBitmapWords : 1u];
  // Word t % 8 of part t / 8 (t < 32) is the OR of the part's records (one
  // per slice).  The loads are taken on every path and ORed only where the
  // words are staged, so that they go out with the plan's loads (with fewer
  // records the last is read again, which the OR absorbs; threads past the
  // 32 words read those of thread 31).
  uint32_t pwr[kSelfPlan && kCiera ? kSlices : 1u];
  if (kSelfPlan && kCiera) {
    const uint32_t t = min(tid, kBitmapWords - 1u);
    const uint64_t rec0 = (uint64_t(c) * kParts + t / kPartBitmapWords) * ws.ss;
#pragma unroll
    for (uint32_t sl = 0; sl < kSlices; sl++)
      pwr[sl] = ws.bitmap[(rec0 + min(sl, ws.ss - 1u)) * kPartBitmapWords + t % kPartBitmapWords];
  }
  // Nothing is written unless the plan is complete and puts the chunk inside
  // the output buffer.
  auto plan_ok = [&](bool plan_failed) {
    return !(plan_failed || begin < table_end(nchunks) || (begin & 127u) != 0u || begin > capacity ||
             capacity - begin < chunk_max_bytes(nc, kCiera ? B : 0u) || esc_chunk > nc || esc_before > esc_chunk ||
             esc_part > esc_chunk - esc_before);
  };
  PlanStart ps;
  if (kSelfPlan) {
    // the window base now; the chunks' offsets after the values are coded
    ps = self_plan_start(nchunks, wg, e0_override, out, out_size, ws);
    e0 = ps.e0;
    if (e0 == kBadE0) {  // the same for every workgroup
      if (tid == 0) ws.err[wg] = uint32_t(CIERA_ERR_ARG);
      return;
    }
  } else {
    begin = reinterpret_cast<const uint64_t*>(out + kHeader)[c];
    esc_before = ws.partesc[c * kParts + h];
    esc_chunk = ws.chunkesc[c];
    esc_part = (last_part ? esc_chunk : ws.partesc[c * kParts + h + 1u]) - esc_before;
    e0 = ws.ctrl->e0;
    const bool plan_failed = ws.ctrl->plan_fail != 0u;
    if (!plan_ok(plan_failed)) {
      if (tid == 0) {
        ws.err[wg] = uint32_t(CIERA_ERR_INTERNAL);
        // after a failed plan the stream must not pass for one: no size, no magic
        if (plan_failed && wg == 0u) {
          *out_size = 0u;
          *reinterpret_cast<uint64_t*>(out) = 0u;
        }
      }
      return;
    }
  }
  const uint32_t bias = ((1u - e0) & 0xFFFFu) * 0x00010001u;
  for (uint32_t i = tid; i < 3u * kStage / 16u; i += kPartThreads)
    reinterpret_cast<uint4*>(s_planes)[i] = make_uint4(0u, 0u, 0u, 0u);

  uint32_t nch = 0, nb = 0;
  if (kCiera) {
    const uint32_t* pw = ws.bitmap + uint64_t(c) * kBitmapWords;
    if (kSelfPlan) {
      uint32_t pw_l = 0u;
#pragma unroll
      for (uint32_t sl = 0; sl < kSlices; sl++) pw_l |= pwr[sl];
      if (tid < kBitmapWords) s_pw[tid] = pw_l;
      __syncthreads();
      pw = s_pw;
    }
    if (tid < 64u) stage_bitmap((tid < kBitmapWords) ? chunk_bitmap_word(pw, tid, B) : 0u, s_bits, s_rank);
    nb = (nc + B - 1u) >> log2B;
  }
  __syncthreads();  // staging cleared, bitmap staged
  if (kCiera) nch = s_rank[kBitmapWords - 1] + __popc(s_bits[kBitmapWords - 1]);
  ChunkGeom g = chunk_geom(begin, nc, kCiera, nch, B);  // self-planned: recomputed once the offset is known
  const uint32_t pb = uint32_t(g.plane_bytes);
  // Plane bytes this part stages and writes.  zip3: one byte per unit, so the
  // part owns bytes [pu0, pu0 + kPartUnits) of each plane (padding included).
  // ciera: the slots of the part's units in changed blocks, [S_h, S_next);
  // the last part also owns the padding after the chunk's last slot.  Every
  // bound is a multiple of 8.
  // A slice owns the slots of its own units, [S(u0), S(u0 + kRange)).
  const uint32_t s_h = kCiera ? coded_before(u0, s_bits, s_rank, log2B, nb, nch) : u0;
  const uint32_t s_next = kCiera ? (!(last_part && final_slice) ? coded_before(u0 + kRange, s_bits, s_rank, log2B, nb, nch)
                                                                : nch * (B / 8u))
                                 : u0 + kRange;

  // A slice's first escape: the part's escapes before u0 (values of coded
  // units whose code is 0), from the plan (below), or counted from the units
  // loaded above.
  uint32_t zb = 0;
  if (kS > 1u && !counted) {
    uint32_t z = 0;
#pragma unroll
    for (uint32_t k = 0; k < kEarly; k++) {
      const uint32_t u = pu0 + k * kPartThreads + tid;
      if (u >= u0 || u >= nunits) continue;
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
        for (int i = 0; i < 4; i++) cp[i] = code_pair(exp_pair(ve[k].w[i]), bias);
        const uint32_t p = unit_planes(cp);
        z += __popc(~(p | (p >> 8) | (p >> 16)) & vmask);
      }
    }
    zb = part_sum_u32(z, s_zw);
  }

  // Code every unit: sign+mantissa bytes straight to HBM (self-planned: held
  // until the offset is known), plane bytes into LDS.
  uint32_t cnt[kU], base[kU], emask[kU];
  uint2 smb[kSelfPlan ? kU : 1u];
#pragma unroll
  for (uint32_t j = 0; j < kU; j++) {
    const uint32_t u = u0 + j * kPartThreads + tid;
    cnt[j] = 0u;
    emask[j] = 0u;
    if (kSelfPlan) smb[j] = unit_sm(v[j]);
    if (u < nunits) {
      if (!kSelfPlan) *reinterpret_cast<uint2*>(out + g.sm + 8ull * u) = unit_sm(v[j]);
      bool coded = true;
      uint32_t pbyte = u;
      if (kCiera) {
        const uint32_t blk = (8u * u) >> log2B;
        coded = (s_bits[blk >> 5] >> (blk & 31u)) & 1u;
        pbyte = coded_before(u, s_bits, s_rank, log2B, nb, nch);
      }
      if (coded) {
        const uint32_t valid = min(8u, nc - 8u * u);
        const uint32_t vmask = (valid == 8u) ? 0xFFu : ((1u << valid) - 1u);
        uint32_t cp[4];
#pragma unroll
        for (int i = 0; i < 4; i++) cp[i] = code_pair(exp_pair(v[j].w[i]), bias);
        const uint32_t p = unit_planes(cp) & (vmask * 0x010101u);
        const uint32_t at = pbyte - s_h;
        s_planes[at] = uint8_t(p);
        s_planes[kStage + at] = uint8_t(p >> 8);
        s_planes[2u * kStage + at] = uint8_t(p >> 16);
        emask[j] = ~(p | (p >> 8) | (p >> 16)) & vmask;
        cnt[j] = __popc(emask[j]);
      }
    }
  }
  const uint32_t pesc = part_escape_scan<kU, false>(cnt, base, s_tot);  // its barriers also complete the plane staging
  if (kSelfPlan) {
    // The escapes need no stream position: staged now; the plan's second
    // step (its barriers complete the staging) gives the offsets.
    stage_escapes(v, emask, base, s_esc);
    const SelfPlan sp = self_plan_finish(n, nchunks, c, h, slice, h == 0u && slice == 0u, wg, kCiera ? B : 0u, ps,
                                         out, out_size, ws);
    begin = sp.begin;
    esc_before = sp.esc_before;
    esc_chunk = sp.esc_chunk;
    esc_part = sp.esc_part;
    esc_slice = sp.esc_slice;
    esc_slice_before = sp.esc_slice_before;
    if (counted) zb = esc_slice_before;
    if (!plan_ok(false)) {
      if (tid == 0) ws.err[wg] = uint32_t(CIERA_ERR_INTERNAL);
      return;
    }
    g = chunk_geom(begin, nc, kCiera, nch, B);
#pragma unroll
    for (uint32_t j = 0; j < kU; j++) {
      const uint32_t u = u0 + j * kPartThreads + tid;
      if (u < nunits) *reinterpret_cast<uint2*>(out + g.sm + 8ull * u) = smb[j];
    }
  }
  // The count must match what the plan read off the histograms (a slice: its
  // escapes and those before it stay within the part's, the last slice's end
  // where the part's do, and one the plan counted has its planned count); a
  // mismatch would overrun the escape section, so no escapes are written and
  // the error word reports it.
  const bool esc_ok = (final_slice ? zb + pesc == esc_part : zb + pesc <= esc_part) && (!counted || pesc == esc_slice);
  if (tid == 0) ws.err[wg] = esc_ok ? 0u : uint32_t(CIERA_ERR_INTERNAL);
  // planes: LDS -> HBM in 8-byte pieces over the owned range, clipped to the
  // padded plane length
  const uint32_t own_hi = min(s_next, pb);
  const uint32_t own = own_hi > s_h ? own_hi - s_h : 0u;
  for (uint32_t i = tid; i < 3u * (own / 8u); i += kPartThreads) {
    const uint32_t b = i / (own / 8u);
    const uint32_t off = 8u * (i - b * (own / 8u));
    const uint2 val = *reinterpret_cast<const uint2*>(s_planes + b * kStage + off);
    *reinterpret_cast<uint2*>(out + g.plane + b * pb + s_h + off) = val;
  }
  // escapes of this range: [esc_before + zb, + pesc) of the chunk's section
  const uint64_t esc_at = g.esc + esc_before + zb;
  if (esc_ok) {
    if (!kSelfPlan) {
      stage_escapes(v, emask, base, s_esc);
      __syncthreads();
    }
    lds_to_global(out + esc_at, s_esc, pesc, tid, kPartThreads);
  }
  if (last_part && final_slice) {
    // zero padding after each section's data, and the bitmap
    zero_fill(out, g.sm + 8ull * nunits, g.bitmap, kPartThreads);
    if (kCiera && tid < kBitmapWords) *reinterpret_cast<uint32_t*>(out + g.bitmap + 4u * tid) = s_bits[tid];
    if (kCiera)
      for (uint32_t b = 0; b < 3u; b++) zero_fill(out, g.plane + b * pb + s_next, g.plane + (b + 1u) * pb, kPartThreads);
    if (esc_chunk <= kChunk) zero_fill(out, g.esc + esc_chunk, g.esc + pad128(esc_chunk), kPartThreads);
  }
}

// ------------------------------------------------------------------ single-read encode
// With the window base known in advance (a byte in device memory, e.g. byte
// 7 of the previous iteration's stream), encode needs no variance pass and
// reads x once.  The window rule of the ZipCCL digest (section 3.1) sets E0
// from the tensor's sigma; which tensor's sigma is the caller's choice here.
// k_prep1 writes the header and clears the look-back words.  k_write1 codes
// one part, publishes its escape count and reads those of its chunk's other
// parts, so that every part knows the chunk's size.  Every part then looks
// back over the earlier chunks (decoupled look-back: a chunk's size follows
// from its parts' published counts) for the chunk's offset, and the chunk's
// last part publishes the chunk's inclusive prefix.
// Every value passed between workgroups sits in the one word that carries its
// ready flag, so relaxed device-scope atomics suffice (no cache-wide
// acquire/release).  A part waits only on its own chunk's parts and on
// earlier chunks: the lowest unfinished chunk always has all of its parts
// dispatched, so every wait ends; each is bounded as well and ends in
// CIERA_ERR_INTERNAL.
constexpr uint64_t kFlagSize = 1ull << 62;  // look-back only: a predecessor's size, not a prefix
constexpr uint64_t kFlagIncl = 2ull << 62;
constexpr uint64_t kFlagFail = 3ull << 62;  // the chunk's last part gave up a wait: no offset follows
constexpr uint64_t kValMask = (1ull << 62) - 1u;
constexpr uint32_t kDoneShift = 40u;           // ctrl->done_esc: chunks << 40 | escapes
constexpr uint64_t kMaxSingleReadN = 1ull << 39;  // keeps both fields of done_esc in range

// A part's published word: bit 31 ready, bits 15..30 a 16-bit field, bits
// 0..14 the part's escapes (at most 16,384).  The field is 0 in zip3 mode;
// in ciera mode, with B <= 512 the part's changed blocks (at most 256), with
// 1024 <= B <= 16384 the part's block bits (at most 16), with B > 16384 bit
// 0 = some value of the part changed (its share of the block).
// Pause between two polls of another workgroup's word in the single-read
// encode (s_sleep units of 64 cycles): each poll is a round trip past the
// XCD's L2; polling 16 times less often made k_write1 2 % faster on the
// 10^9-value stress buffer.
constexpr int kPollSleep = 16;
constexpr uint32_t kPartReady = 1u << 31;
constexpr uint32_t kEscBits = 15u;
__device__ inline uint32_t word_esc(uint32_t w) { return w & ((1u << kEscBits) - 1u); }
__device__ inline uint32_t word_field(uint32_t w) { return (w >> kEscBits) & 0xFFFFu; }

// A chunk's layout from its parts' words: its changed blocks and escapes,
// per part the escapes and plane bytes before it in the chunk, and whether
// it codes its values (a part inside a block that spans several parts codes
// them only if some part of the block changed).
struct ChunkCounts {
  uint32_t nch, esc, coded;  // coded: bit h for part h
  uint32_t esc_before[kParts], slot_before[kParts];
};
__device__ inline ChunkCounts chunk_counts(const uint32_t (&w)[kParts], bool ciera, uint32_t log2B) {
  ChunkCounts k;
  k.nch = k.esc = k.coded = 0u;
  const uint32_t B = 1u << log2B;
  if (!ciera || B <= kPartValues) {
    uint32_t slots = 0;
#pragma unroll
    for (uint32_t h = 0; h < kParts; h++) {
      k.esc_before[h] = k.esc;
      k.slot_before[h] = slots;
      k.esc += word_esc(w[h]);
      const uint32_t f = word_field(w[h]);
      const uint32_t nb = !ciera ? 0u : (B <= 512u ? f : uint32_t(__popc(f)));
      k.nch += nb;
      slots += nb * (B / 8u);
      k.coded |= 1u << h;
    }
  } else {
    const uint32_t ppb = B / kPartValues;  // parts per block: 2 or 4
    uint32_t rank = 0;
#pragma unroll
    for (uint32_t h = 0; h < kParts; h++) {
      const uint32_t first = h / ppb * ppb;
      uint32_t any = 0;
      for (uint32_t q = first; q < first + ppb; q++) any |= word_field(w[q]) & 1u;
      if (h == first && any) rank++;  // this block's rank + 1 among the changed blocks
      k.slot_before[h] = any ? (rank - 1u) * (B / 8u) + (h - first) * (kPartValues / 8u) : 0u;
      k.esc_before[h] = k.esc;
      if (any) {
        k.coded |= 1u << h;
        k.esc += word_esc(w[h]);
      }
    }
    k.nch = rank;
  }
  return k;
}

// Stream bytes of a chunk of nc values.
__device__ inline uint64_t chunk_bytes(uint32_t nc, bool ciera, uint32_t log2B, uint32_t nch, uint32_t esc) {
  const uint64_t planes = ciera ? (uint64_t(nch) << log2B) / 8u : cdiv(nc, 8u);
  return pad128(nc) + (ciera ? 128u : 0u) + 3u * pad128(planes) + pad128(esc);
}

__global__ __launch_bounds__(kThreads) void k_prep1(uint64_t n, uint64_t nchunks, uint32_t B,
                                                    const uint8_t* __restrict__ d_e0, uint8_t* __restrict__ out,
                                                    uint64_t* __restrict__ out_size, Ws ws) {
  // every workgroup clears its share of the look-back words; workgroup 0
  // also writes the header and the control words
  const uint32_t tid = threadIdx.x;
  const uint64_t first = uint64_t(blockIdx.x) * kThreads + tid, stride = uint64_t(gridDim.x) * kThreads;
  uint64_t* hd = reinterpret_cast<uint64_t*>(out);
  uint64_t* table = reinterpret_cast<uint64_t*>(out + kHeader);
  const uint64_t base = table_end(nchunks);
  const uint32_t e0 = d_e0[0];
  const bool ok = e0 <= kMaxE0;
  for (uint64_t i = first; i < nchunks * kParts; i += stride)
    ws.pcount[(i / kParts) * kPcountStride + i % kParts] = 0u;
  for (uint64_t i = first; i < nchunks; i += stride) ws.cstat[i * kCstatStride] = 0u;
  if (blockIdx.x != 0u) return;
  if (tid == 0) {
    ws.ctrl->done_esc = 0u;
    ws.ctrl->done_nch = 0u;
    ws.ctrl->spec = 0u;
    ws.ctrl->spec_fail = 0u;
    ws.ctrl->e0 = ok ? e0 : kBadE0;
    ws.ctrl->n_err_slots = nchunks ? nchunks * kParts : 1u;
    if (nchunks == 0u) ws.err[0] = ok ? 0u : uint32_t(CIERA_ERR_ARG);
  }
  if (!ok) {
    // An invalid window base: the stream gets only its first header word,
    // whose E0 byte keeps the bad value, so that neither a decoder nor a
    // next encode that takes its window base from byte 7 accepts it.
    if (tid == 0) {
      hd[0] = uint64_t(e0) << 56;
      *out_size = 0u;
    }
    return;
  }
  // the padding words after the chunk table and the escape index
  for (uint64_t i = 2u * nchunks + 1u + tid; i < (base - kHeader) / 8u; i += kThreads) table[i] = 0u;
  if (tid == 0) {
    const uint32_t magic = B ? 0x52454943u /* "CIER" */ : 0x3350495Au /* "ZIP3" */;
    hd[0] = uint64_t(magic) | (1ull << 32) | (uint64_t(B ? 1u : 0u) << 48) | (uint64_t(e0) << 56);
    hd[1] = n;
    hd[2] = uint64_t(B) | (uint64_t(kChunk) << 32);
    hd[3] = nchunks;
    hd[5] = 0u;
    for (int i = 7; i < 16; i++) hd[i] = 0u;
    if (nchunks == 0u) {
      hd[4] = base;
      hd[6] = 0u;
      table[0] = base;
      *out_size = base;
    }
  }
}

// Stream bytes of the chunks before c (wave 0, 64 predecessors at a time).
// A predecessor's status word holds its inclusive prefix once its last part
// has looked back (the search ends there), else its size as soon as one of
// its parts knows it (all four parts' counts are in), else nothing yet.
// Returns false if a wait did not end.
__device__ inline bool chunk_lookback(const Ws& ws, uint64_t c, uint64_t& pb) {
  const uint32_t lane = lane_id();
  pb = 0;
  int64_t top = int64_t(c) - 1;
  uint32_t spins = 0;
  while (top >= 0) {
    const int64_t k = top - int64_t(lane);
    const uint64_t st = (k >= 0) ? load_relaxed(&ws.cstat[uint64_t(k) * kCstatStride]) : kFlagIncl;
    const uint64_t flag = st & ~kValMask;
    if (__ballot(flag == kFlagFail) != 0u) return false;
    if (__ballot(flag == 0u) != 0u) {
      if (++spins > ws.spin_limit) return false;
      __builtin_amdgcn_s_sleep(kPollSleep);
      continue;
    }
    const uint64_t incl = __ballot(flag == kFlagIncl);
    if (incl != 0u) {
      const uint32_t first = uint32_t(__builtin_ctzll(incl));
      pb += wave_sum_u64(lane <= first ? (st & kValMask) : 0u);
      return true;
    }
    pb += wave_sum_u64(st & kValMask);
    top -= 64;
  }
  return true;
}

// Part index of workgroup b: XCD x = b mod 8 takes chunks x, x + 8, x + 16,
// ... with their parts in order; the chunks past the last full group of 8
// keep the plain mapping.
__device__ inline uint32_t single_part_of(uint32_t b, uint32_t nchunks) {
  const uint32_t grouped = nchunks / kXcds * kXcds * kParts;
  if (b >= grouped) return b;
  const uint32_t x = b % kXcds, slot = b / kXcds;
  return ((slot / kParts) * kXcds + x) * kParts + slot % kParts;
}

// One part of a chunk.  ciera mode: the part also compares its exponents with
// the sender cache, rewrites the units that differ, and codes only the
// values of its changed blocks (a block that spans several parts: once the
// chunk's words show some part of it changed).
// kSigma: the speculative encode's write, with the window base a hint (e.g.
// the previous iteration's): the part also adds its variance sums exactly as
// k_stats does and leaves k_stats' records (sums, change bits), so that
// k_sums and k_check can tell whether the hint is the window the variance
// gives, and the fallback launches can redo the encode if not; with an
// out-of-range hint it writes only those records and the cache.
template <bool kCiera, bool kSigma = false>
__global__ __launch_bounds__(kPartThreads) void k_write1(const uint16_t* __restrict__ x, uint64_t n, uint64_t nchunks,
                                                         uint32_t log2B, uint8_t* __restrict__ cache,
                                                         uint8_t* __restrict__ out, uint64_t* __restrict__ out_size,
                                                         Ws ws) {
  __shared__ __attribute__((aligned(16))) uint8_t s_planes[3u * kStage];
  __shared__ __attribute__((aligned(16))) uint8_t s_esc[kPartEscStage];
  __shared__ uint32_t s_tot[kUPT * kPartWaves + 1];
  __shared__ uint32_t s_pbits[kPartBitmapWords];  // ciera: the part's block bits (B > 16384: bit 0, its share)
  __shared__ uint64_t s_begin;
  __shared__ uint32_t s_before, s_slot0, s_nch, s_coded, s_err;
  __shared__ double s_vs1[kSigma ? kPartWaves : 1u], s_vs2[kSigma ? kPartWaves : 1u];
  __shared__ uint32_t s_vnf[kSigma ? kPartWaves : 1u];
  const uint32_t tid = threadIdx.x;
  const uint32_t lane = lane_id(), wave = tid >> 6;
  // Workgroups are dealt round-robin over the chip's 8 XCDs; the four parts of
  // a chunk go to one XCD, one after the other, so that they are dispatched
  // together and wait on each other only briefly.
  const uint32_t wg = single_part_of(blockIdx.x, uint32_t(nchunks));
  const uint64_t c = wg / kParts;
  const uint32_t h = wg % kParts;
  const bool last_part = h + 1u == kParts;
  const uint64_t start = c * kChunk;
  const uint32_t nc = uint32_t(min(uint64_t(kChunk), n - start));
  const uint32_t nunits = (nc + 7u) / 8u;
  const uint32_t pu0 = h * kPartUnits;
  const uint32_t B = kCiera ? (1u << log2B) : 0u;
  const uint32_t e0 = ws.ctrl->e0;
  if (!kSigma && e0 == kBadE0) {  // the same for every workgroup: none waits on another
    if (tid == 0) ws.err[wg] = uint32_t(CIERA_ERR_ARG);
    return;
  }

  // Load the part (and its cache bytes) first: all loads go out before any is used.
  Unit v[kUPT];
  uint2 old[kUPT];
  const bool full = 8u * (pu0 + kPartUnits) <= nc;
  if (full) {
#pragma unroll
    for (uint32_t j = 0; j < kUPT; j++) v[j] = load_unit(x, start + 8ull * (pu0 + j * kPartThreads + tid), 8u);
    if (kCiera) {
#pragma unroll
      for (uint32_t j = 0; j < kUPT; j++)
        old[j] = *reinterpret_cast<const uint2*>(cache + start + 8ull * (pu0 + j * kPartThreads + tid));
    }
  } else {
#pragma unroll
    for (uint32_t j = 0; j < kUPT; j++) {
      const uint32_t u = pu0 + j * kPartThreads + tid;
      v[j].w[0] = v[j].w[1] = v[j].w[2] = v[j].w[3] = 0u;
      old[j] = make_uint2(0u, 0u);
      if (u < nunits) {
        v[j] = load_unit(x, start + 8ull * u, min(8u, nc - 8u * u));
        if (kCiera) old[j] = load_bytes8(cache + start + 8ull * u, min(8u, nc - 8u * u));
      }
    }
  }
  // kSigma: the variance sums' shift, read after the part's loads are out
  const double shift = kSigma ? stats_shift(x[0]) : 0.0;
  // From here on a unit lives as its exponent bytes and its sign+mantissa
  // bytes (half the registers of the loaded words, held until the stores).
  // kSigma: each unit first adds to the variance sums, as in k_stats.
  uint2 ex[kUPT], smb[kUPT];
  double s1 = 0.0, s2 = 0.0;
  uint32_t nf = 0;
#pragma unroll
  for (uint32_t j = 0; j < kUPT; j++) {
    if (kSigma) {
      const uint32_t u = pu0 + j * kPartThreads + tid;
      if (full || u < nunits) stats_unit(v[j], full ? 8u : min(8u, nc - 8u * u), shift, s1, s2, nf);
    }
    ex[j] = unit_exponents(v[j]);
    smb[j] = unit_sm(v[j]);
  }
  if (kSigma && !(__builtin_isfinite(s1) && __builtin_isfinite(s2))) {
    // a non-finite value: the units again with the finiteness test, the
    // values rebuilt from their bytes
    s1 = 0.0;
    s2 = 0.0;
    nf = 0;
#pragma unroll
    for (uint32_t j = 0; j < kUPT; j++) {
      const uint32_t u = pu0 + j * kPartThreads + tid;
      if (u < nunits) stats_checked(unit_join(smb[j], ex[j]), min(8u, nc - 8u * u), shift, s1, s2, nf);
    }
  }
  const uint32_t bias = ((1u - e0) & 0xFFFFu) * 0x00010001u;
  for (uint32_t i = tid; i < 3u * kStage / 16u; i += kPartThreads)
    reinterpret_cast<uint4*>(s_planes)[i] = make_uint4(0u, 0u, 0u, 0u);
  if (kCiera && tid < kPartBitmapWords) s_pbits[tid] = 0u;
  __syncthreads();  // staging cleared

  // ciera: exponents against the cache; the units that differ are rewritten,
  // and a wave ballot gives the changed blocks among the wave's 64 units
  // (lanes [kL, kL + L) hold block k for L = B / 8 up to 64; from B = 512 on
  // the 64 units lie in one block), set in s_pbits by one atomic per wave.
  // Blocks count from the part's start; with B > 16384 the part is one share.
  if (kCiera) {
    const uint32_t L = (B >= 512u) ? 64u : B / 8u;
    const uint64_t gmask = (L >= 64u) ? ~0ull : ((1ull << L) - 1u);
    const uint32_t lb = min(log2B, 14u);  // the part's blocks are min(B, 16384) values long
#pragma unroll
    for (uint32_t j = 0; j < kUPT; j++) {
      const uint32_t u = pu0 + j * kPartThreads + tid;
      bool diff = false;
      uint32_t cnt = 0u;
      uint2 e = make_uint2(0u, 0u);
      if (u < nunits) {
        cnt = min(8u, nc - 8u * u);
        e = ex[j];
        const uint64_t keep = (cnt == 8u) ? ~0ull : ((1ull << (8u * (cnt & 7u))) - 1u);
        diff = (((uint64_t(e.y ^ old[j].y) << 32) | (e.x ^ old[j].x)) & keep) != 0u;
      }
      const uint64_t m = __ballot(diff);
      if (m != 0u) {
        if (u < nunits && line_has_change(m)) store_bytes8(cache + start + 8ull * u, cnt, e);
        const uint32_t lbw = (8u * (j * kPartThreads + 64u * wave)) >> lb;  // the wave's first block in the part
        uint32_t bits = 0;
        for (uint32_t k = 0; k < 64u / L; k++) bits |= ((m >> (k * L)) & gmask) ? (1u << k) : 0u;
        if (lane == 0u) atomicOr(&s_pbits[lbw >> 5], bits << (lbw & 31u));
      }
    }
    __syncthreads();  // s_pbits complete
  }
  if (kSigma) {
    // the part's records in k_stats' form: variance sums (waves in order)
    // and change bits
    s1 = wave_sum(s1);
    s2 = wave_sum(s2);
    nf = wave_sum_u32(nf);
    if (lane == 0u) {
      s_vs1[wave] = s1;
      s_vs2[wave] = s2;
      s_vnf[wave] = nf;
    }
    __syncthreads();
    if (tid == 0) {
      double a = 0.0, bsum = 0.0;
      uint32_t m = 0;
#pragma unroll
      for (uint32_t w = 0; w < kPartWaves; w++) {
        a += s_vs1[w];
        bsum += s_vs2[w];
        m += s_vnf[w];
      }
      Partial p;
      p.s1 = a;
      p.s2 = bsum;
      p.nf = m;
      p.nch = 0u;
      p.coded = 0u;
      p.pad = 0u;
      ws.partial[wg] = p;
    }
    if (kCiera && tid < kPartBitmapWords) ws.bitmap[uint64_t(wg) * kPartBitmapWords + tid] = s_pbits[tid];
    if (e0 == kBadE0) {  // the same for every workgroup: the fallback writes the stream
      if (tid == 0) {
        ws.err[wg] = 0u;
        ws.ctrl->spec_fail = 1u;
      }
      return;
    }
  }
  // the part's changed blocks; lane k < kPartBitmapWords holds those before
  // bitmap word k
  uint32_t pnch = 0, prank_l = 0;
  if (kCiera) {
    const uint32_t pc = lane < kPartBitmapWords ? uint32_t(__popc(s_pbits[lane])) : 0u;
    const uint32_t incl = wave_incl_scan(pc);
    prank_l = incl - pc;
    pnch = uint32_t(__builtin_amdgcn_readlane(int(incl), int(kPartBitmapWords - 1u)));
  }

  // Code every unit that is coded: plane bytes into LDS at the unit's plane
  // byte within the part's slots (zip3: the unit's own byte), escape masks.
  uint32_t cnt[kUPT], base[kUPT], em4[kUPT / 4u] = {};  // escape masks, unit j in byte j % 4 of em4[j / 4]
#pragma unroll
  for (uint32_t j = 0; j < kUPT; j++) {
    const uint32_t u = pu0 + j * kPartThreads + tid;
    const uint32_t ul = u - pu0;
    cnt[j] = 0u;
    bool coded = true;
    uint32_t at = ul;
    if (kCiera && B <= kPartValues) {
      const uint32_t upb_log = log2B - 3u;  // units per block
      const uint32_t blk = ul >> upb_log;
      const uint32_t word = s_pbits[blk >> 5];
      const uint32_t before = uint32_t(__shfl(int(prank_l), int(blk >> 5)));  // changed blocks in the words before blk's
      coded = (word >> (blk & 31u)) & 1u;
      at = ((before + __popc(word & ((1u << (blk & 31u)) - 1u))) << upb_log) + (ul & ((1u << upb_log) - 1u));
    }
    if (u < nunits && coded) {
      const uint32_t valid = min(8u, nc - 8u * u);
      const uint32_t vmask = (valid == 8u) ? 0xFFu : ((1u << valid) - 1u);
      uint32_t cp[4];
#pragma unroll
      for (int i = 0; i < 4; i++)
        cp[i] = code_pair(perm(0u, i < 2 ? ex[j].x : ex[j].y, (i & 1) ? 0x0C030C02u : 0x0C010C00u), bias);
      const uint32_t p = unit_planes(cp) & (vmask * 0x010101u);
      s_planes[at] = uint8_t(p);
      s_planes[kStage + at] = uint8_t(p >> 8);
      s_planes[2u * kStage + at] = uint8_t(p >> 16);
      const uint32_t em = ~(p | (p >> 8) | (p >> 16)) & vmask;
      em4[j / 4u] |= em << (8u * (j % 4u));
      cnt[j] = __popc(em);
    }
  }
  const uint32_t pesc = part_escape_scan(cnt, base, s_tot);  // its barriers also complete the plane staging
  uint32_t field = 0u;
  if (kCiera) field = (B <= 512u) ? pnch : (B <= kPartValues ? s_pbits[0] : (s_pbits[0] & 1u));
  if (tid == 0) store_relaxed(&ws.pcount[c * kPcountStride + h], kPartReady | (field << kEscBits) | pesc);
  // the escapes need no stream position: staged while the part waits for it
  stage_escapes_ex(ex, em4, base, s_esc);

  // Stream position (wave 0).
  if (tid < 64u) {
    uint32_t err = 0u;
    // the words of the chunk's four parts: lane l < 4 reads part l's
    uint32_t w_l = 0u;
    for (uint32_t spins = 0;; spins++) {
      w_l = (lane < kParts) ? load_relaxed(&ws.pcount[c * kPcountStride + lane]) : kPartReady;
      if (__ballot(!(w_l & kPartReady)) == 0u) break;
      if (spins > ws.spin_limit) {
        err = CIERA_ERR_INTERNAL;
        break;
      }
      __builtin_amdgcn_s_sleep(2 * kPollSleep);
    }
    uint32_t w[kParts];
#pragma unroll
    for (uint32_t q = 0; q < kParts; q++) w[q] = uint32_t(__builtin_amdgcn_readlane(int(w_l), int(q)));
    const ChunkCounts cc = chunk_counts(w, kCiera, log2B);
    const uint64_t size = chunk_bytes(nc, kCiera, log2B, cc.nch, cc.esc);
    const uint64_t tbl = table_end(nchunks);
    uint64_t* table = reinterpret_cast<uint64_t*>(out + kHeader);
    uint64_t pb = 0;
    uint64_t* cst = &ws.cstat[c * kCstatStride];
    // Every part publishes the chunk's size (the same value; the maximum
    // keeps an inclusive prefix that is already there, its flag being the
    // larger).  The last part looks back for the chunk's offset and publishes
    // the inclusive prefix; the others wait for it on the chunk's own word.
    if (!err && lane == 0u)
      atomicMax(reinterpret_cast<unsigned long long*>(cst), (unsigned long long)(kFlagSize | size));
    if (last_part) {
      if (!err && !chunk_lookback(ws, c, pb)) err = CIERA_ERR_INTERNAL;
    } else if (!err) {
      // The last part publishes the inclusive prefix, or kFlagFail if it gave
      // up a wait (its size may then come from incomplete counts and must not
      // be subtracted from); a prefix below the chunk's own size is refused too.
      uint64_t st = 0;
      for (uint32_t spins = 0;; spins++) {
        st = shfl_u64(load_relaxed(cst), 0u);  // lane 0's read: one decision for the wave
        if ((st & ~kValMask) >= kFlagIncl) break;
        if (spins > ws.spin_limit) break;
        __builtin_amdgcn_s_sleep(kPollSleep);
      }
      if ((st & ~kValMask) == kFlagIncl && (st & kValMask) >= size)
        pb = (st & kValMask) - size;
      else
        err = CIERA_ERR_INTERNAL;
    }
    if (last_part) {
      if (lane == 0u) {
        // published even after a failed wait (as a failure), so that no later
        // wait lasts forever and no other part takes an offset from it
        store_relaxed(cst, err ? kFlagFail : (kFlagIncl | (pb + size)));
        table[c] = tbl + pb;
        table[nchunks + 1u + c] = (uint64_t(cc.esc_before[1]) << 16) | (uint64_t(cc.esc_before[2]) << 32) |
                                  (uint64_t(cc.esc_before[3]) << 48);
        if (c + 1u == nchunks) {
          uint64_t* hd = reinterpret_cast<uint64_t*>(out);
          table[nchunks] = tbl + pb + size;
          hd[4] = tbl + pb + size;
          *out_size = tbl + pb + size;
        }
        // The chunk that finishes last writes the totals.  Each chunk adds its
        // changed blocks before it counts itself done: the second atomic
        // takes an operand from the first's result, so it is issued only
        // once the first is performed.
        uint64_t dep = 0u;
        if (kCiera) dep = atomicAdd(reinterpret_cast<unsigned long long*>(&ws.ctrl->done_nch), cc.nch) >> 63;
        const uint64_t old_d = atomicAdd(reinterpret_cast<unsigned long long*>(&ws.ctrl->done_esc),
                                         ((1ull << kDoneShift) | cc.esc) + dep);
        if ((old_d >> kDoneShift) + 1u == nchunks) {
          uint64_t* hd = reinterpret_cast<uint64_t*>(out);
          hd[6] = (old_d & ((1ull << kDoneShift) - 1u)) + cc.esc;
          if (kCiera) hd[5] = load_relaxed(&ws.ctrl->done_nch);
        }
      }
    }
    if (lane == 0u) {
      uint32_t eb = 0, sb = 0;  // part h's entries (constant indices: no private array)
#pragma unroll
      for (uint32_t q = 0; q < kParts; q++) {
        eb = (q == h) ? cc.esc_before[q] : eb;
        sb = (q == h) ? cc.slot_before[q] : sb;
      }
      s_begin = tbl + pb;
      s_before = eb;
      s_slot0 = sb;
      s_nch = cc.nch;
      s_coded = (cc.coded >> h) & 1u;
      s_err = err;
    }
  }
  __syncthreads();
  if (s_err) {
    if (tid == 0) {
      ws.err[wg] = s_err;
      if (kSigma) ws.ctrl->spec_fail = 1u;  // the fallback redoes the encode
    }
    return;
  }
  const uint64_t begin = s_begin;
  const uint32_t esc_before = s_before;
  const uint32_t nch = s_nch;
  const bool coded_part = s_coded != 0u;
  const ChunkGeom g = chunk_geom(begin, nc, kCiera, nch, B);
  const uint32_t pb = uint32_t(g.plane_bytes);
  // sign+mantissa bytes
#pragma unroll
  for (uint32_t j = 0; j < kUPT; j++) {
    const uint32_t u = pu0 + j * kPartThreads + tid;
    if (u < nunits) *reinterpret_cast<uint2*>(out + g.sm + 8ull * u) = smb[j];
  }
  // planes: the part's plane bytes [slot0, slot0 + own) of each plane, clipped
  // to the padded plane length (zip3: bytes [pu0, pu0 + kPartUnits))
  const uint32_t slot0 = kCiera ? s_slot0 : pu0;
  const uint32_t span = !kCiera ? kPartUnits : (!coded_part ? 0u : (B <= kPartValues ? pnch * (B / 8u) : kPartUnits));
  const uint32_t own_hi = min(slot0 + span, pb);
  const uint32_t own = own_hi > slot0 ? own_hi - slot0 : 0u;
  for (uint32_t i = tid; i < 3u * (own / 8u); i += kPartThreads) {
    const uint32_t b = i / (own / 8u);
    const uint32_t off = 8u * (i - b * (own / 8u));
    const uint2 val = *reinterpret_cast<const uint2*>(s_planes + b * kStage + off);
    *reinterpret_cast<uint2*>(out + g.plane + b * pb + slot0 + off) = val;
  }
  // escapes of this part: [esc_before, esc_before + pesc) of the chunk's section
  const uint64_t esc_at = g.esc + esc_before;
  if (coded_part) lds_to_global(out + esc_at, s_esc, pesc, tid, kPartThreads);  // staged before the wait's barrier
  if (kCiera) {
    // the chunk's bitmap: with B <= 512 each part writes its own words; else
    // the last part assembles the (at most two) words, the others zero
    const uint32_t bpp = kPartValues >> min(log2B, 14u);  // blocks per part (1 with B > 16384)
    if (B <= 512u) {
      if (tid < bpp / 32u)
        *reinterpret_cast<uint32_t*>(out + g.bitmap + 4u * (h * (bpp / 32u) + tid)) = s_pbits[tid];
    } else if (last_part && tid < 64u) {
      uint32_t wl = 0u;
      if (lane < kParts) wl = load_relaxed(&ws.pcount[c * kPcountStride + lane]);
      uint64_t bits = 0;
      if (B <= kPartValues) {
#pragma unroll
        for (uint32_t q = 0; q < kParts; q++)
          bits |= uint64_t(word_field(uint32_t(__builtin_amdgcn_readlane(int(wl), int(q))))) << (q * bpp);
      } else {
        const uint32_t ppb = B / kPartValues;
#pragma unroll
        for (uint32_t q = 0; q < kParts; q++)
          bits |= uint64_t(word_field(uint32_t(__builtin_amdgcn_readlane(int(wl), int(q)))) & 1u) << (q / ppb);
      }
      if (tid < 2u) *reinterpret_cast<uint32_t*>(out + g.bitmap + 4u * tid) = uint32_t(bits >> (32u * tid));
    }
  }
  if (last_part) {
    // zero padding after each section's data (and the bitmap's unused words)
    const uint32_t esc_chunk = esc_before + (coded_part ? pesc : 0u);
    zero_fill(out, g.sm + 8ull * nunits, g.bitmap, kPartThreads);
    if (kCiera) {
      const uint32_t used = (B <= 512u) ? (kChunk >> log2B) / 8u : 8u;  // bitmap bytes written above
      zero_fill(out, g.bitmap + used, g.plane, kPartThreads);
      const uint32_t slots = uint32_t((uint64_t(nch) << log2B) / 8u);
      for (uint32_t b = 0; b < 3u; b++) zero_fill(out, g.plane + b * pb + slots, g.plane + (b + 1u) * pb, kPartThreads);
    }
    if (esc_chunk <= kChunk) zero_fill(out, g.esc + esc_chunk, g.esc + pad128(esc_chunk), kPartThreads);
  }
  if (tid == 0) ws.err[wg] = 0u;
}

// ------------------------------------------------------------------ k_decode
// Escape bytes a decoding part stages in LDS: from the 16-byte boundary at or
// below its first escape, all of its escapes (at most kPartUnits * 8, after at
// most 15 bytes of earlier parts').  The LDS array has 16 spare bytes for the
// 12-byte reads of merge_escapes.
constexpr uint32_t kEscStage = kPartUnits * 8u + 16u;
constexpr uint32_t kDecodeBatchMax = CIERA_DECODE_BATCH_MAX;  // streams per batch decode
static_assert(kEscStage % 16u == 0u, "escape staging");

// Put a unit's escape bytes into e: the k-th set bit of emask (a code-0
// byte) takes the k-th byte from byte a of the staged escapes.  Byte
// selectors for v_perm from the escape ranks (a byte-wise prefix count of
// emask's bits), no loop.
__device__ inline uint2 merge_escapes(uint2 e, uint32_t emask, const uint8_t* s_esc, uint32_t a) {
  const uint32_t* w = reinterpret_cast<const uint32_t*>(s_esc + (a & ~3u));
  const uint32_t sh = a & 3u;
  const uint32_t w0 = w[0], w1 = w[1], w2 = w[2];
  const uint32_t x03 = __builtin_amdgcn_alignbyte(w1, w0, sh);  // the unit's escape bytes 0..3
  const uint32_t x47 = __builtin_amdgcn_alignbyte(w2, w1, sh);  // 4..7
  const uint32_t mlo = spread4(emask & 15u), mhi = spread4(emask >> 4);
  const uint32_t r4 = __popc(emask & 15u);  // escapes among values 0..3
  const uint32_t src_hi = (r4 == 4u) ? x47 : __builtin_amdgcn_alignbyte(x47, x03, r4);
  // selector byte k: the escape's rank (0..3) in the source word, or 4 + k to
  // keep e's byte k
  const uint32_t sel_lo = bfi(mlo * 0xFFu, mlo * 0x01010100u, 0x07060504u);
  const uint32_t sel_hi = bfi(mhi * 0xFFu, mhi * 0x01010100u, 0x07060504u);
  return make_uint2(perm(e.x, x03, sel_lo), perm(e.y, src_hi, sel_hi));
}
constexpr uint32_t kPlaneRounds = (3u * (kStage / 8u) + kPartThreads - 1u) / kPartThreads;

struct DecodePart {
  const uint8_t* in;
  uint16_t* y;
  uint8_t* cache;
  ChunkGeom g;
  uint64_t start;
  uint32_t nc, nunits, pu0, e0, pb, esc_len, sbase, stage_len;
  bool last_with_data;
  uint32_t log2B, nb, nch;
  uint32_t part;    // h: the part's quarter of the chunk
  uint64_t index;   // the chunk's escape index word (four u16)
  uint32_t before;  // escapes of the chunk before the part, from the index
  uint32_t u0;      // the workgroup's first unit: the part's, or its slice's
  uint32_t slot0;   // plane slot of unit u0 (zip3: u0)
  bool final_units; // the workgroup holds the part's last units with data
};

// Decode the units [u0, u0 + kPartUnits / kS) of a part.  kS = 1: the whole
// part.  kS > 1: one slice of it, whose first escape follows from the index
// entry of the part and the code-0 values in the part's slots before u0.
// kFull: every unit of the range holds 8 values, so no per-unit tail
// handling.  Returns the workgroup's status word.
template <bool kCiera, bool kFull, uint32_t kS>
__device__ __attribute__((always_inline)) inline uint32_t decode_part(const DecodePart& p, const uint32_t* s_bits,
                                                                      const uint32_t* s_rank, uint8_t* s_planes,
                                                                      uint8_t* s_esc, uint32_t* s_tot) {
  constexpr uint32_t kU = kUPT / kS;  // units per thread
  __shared__ uint32_t s_zw[kPartWaves];
  const uint32_t tid = threadIdx.x;
  const uint8_t* __restrict__ in = p.in;
  const ChunkGeom& g = p.g;
  // Issue every load before using any: sign+mantissa and, for unchanged
  // blocks, the receiver cache into registers; the part's plane bytes (up to
  // the end of the range) and escapes, staged in LDS.
  uint2 smv[kU], ev[kU];
#pragma unroll
  for (uint32_t j = 0; j < kU; j++) {
    const uint32_t u = p.u0 + j * kPartThreads + tid;
    smv[j] = make_uint2(0u, 0u);
    ev[j] = make_uint2(0u, 0u);
    if (kFull) {
      smv[j] = *reinterpret_cast<const uint2*>(in + g.sm + 8ull * u);
      if (kCiera) {
        // Unchanged blocks read their cache bytes; the units of changed
        // blocks, whose ev the codes replace, read the chunk's first cache
        // bytes instead (one line for the wave).  With the load taken on
        // every path it needs no copy afterwards, and so no wait before the
        // next loads go out.
        const uint32_t blk = (8u * u) >> p.log2B;
        const bool changed = (s_bits[blk >> 5] >> (blk & 31u)) & 1u;
        ev[j] = *reinterpret_cast<const uint2*>(p.cache + p.start + (changed ? 0ull : 8ull * u));
      }
    } else if (u < p.nunits) {
      const uint32_t valid = min(8u, p.nc - 8u * u);
      smv[j] = load_bytes8(in + g.sm + 8ull * u, valid);
      if (kCiera) {
        const uint32_t blk = (8u * u) >> p.log2B;
        if (!((s_bits[blk >> 5] >> (blk & 31u)) & 1u)) ev[j] = load_bytes8(p.cache + p.start + 8ull * u, valid);
      }
    }
  }
  const uint32_t np = p.stage_len / 8u;  // 8-byte pieces per plane, <= kStage / 8
  uint2 st[kPlaneRounds];
#pragma unroll
  for (uint32_t r = 0; r < kPlaneRounds; r++) {
    const uint32_t i = tid + r * kPartThreads;
    if (i < 3u * np) {
      const uint32_t b = uint32_t(i >= np) + uint32_t(i >= 2u * np);  // i < 3 np
      st[r] = *reinterpret_cast<const uint2*>(in + g.plane + b * p.pb + p.sbase + 8u * (i - b * np));
    }
  }
  // Escapes: staged from the 16-byte boundary at or below the part's first
  // escape, as many as the index gives the part (the count is checked against
  // the planes below, before any escape is used).  The section length is a
  // multiple of 128.
  const uint32_t first = min(p.before, p.esc_len);
  const uint32_t esc_lo = first & ~15u;
  const uint32_t next = (p.part + 1u < kParts) ? uint32_t(p.index >> (16u * (p.part + 1u))) & 0xFFFFu : p.esc_len;
  const uint32_t own = min(next > first ? next - first : 0u, kPartUnits * 8u);
  const uint32_t pieces = min((p.esc_len - esc_lo) / 16u, (first - esc_lo + own + 15u) / 16u);
  constexpr uint32_t kEscRounds = 2u;  // pieces loaded before any is used; more are rare
  uint4 se[kEscRounds];
#pragma unroll
  for (uint32_t r = 0; r < kEscRounds; r++) {
    const uint32_t i = tid + r * kPartThreads;
    se[r] = make_uint4(0u, 0u, 0u, 0u);
    if (i < pieces) se[r] = *reinterpret_cast<const uint4*>(in + g.esc + esc_lo + 16u * i);
  }
#pragma unroll
  for (uint32_t r = 0; r < kPlaneRounds; r++) {
    const uint32_t i = tid + r * kPartThreads;
    if (i < 3u * np) {
      const uint32_t b = uint32_t(i >= np) + uint32_t(i >= 2u * np);  // i < 3 np
      *reinterpret_cast<uint2*>(s_planes + b * kStage + 8u * (i - b * np)) = st[r];
    }
  }
#pragma unroll
  for (uint32_t r = 0; r < kEscRounds; r++) {
    const uint32_t i = tid + r * kPartThreads;
    if (i < pieces) reinterpret_cast<uint4*>(s_esc)[i] = se[r];
  }
  for (uint32_t i = tid + kEscRounds * kPartThreads; i < pieces; i += kPartThreads)
    reinterpret_cast<uint4*>(s_esc)[i] = *reinterpret_cast<const uint4*>(in + g.esc + esc_lo + 16u * i);
  __syncthreads();
  uint32_t zb = 0;  // code-0 values of the part before unit u0
  if (kS > 1u) {
    const uint32_t lim = p.slot0 - p.sbase;
    uint32_t z = 0;
    for (uint32_t i = tid; i < lim; i += kPartThreads)
      z += __popc(~(uint32_t(s_planes[i]) | s_planes[kStage + i] | s_planes[2u * kStage + i]) & 0xFFu);
    zb = part_sum_u32(z, s_zw);
  }
  const uint32_t before = p.before + zb;

  uint32_t cnt[kU], base[kU], em4[(kU + 3u) / 4u] = {};  // unit j's escape mask in byte j % 4 of em4[j / 4]
#pragma unroll
  for (uint32_t j = 0; j < kU; j++) {
    const uint32_t u = p.u0 + j * kPartThreads + tid;
    cnt[j] = 0u;
    if (!kFull && u >= p.nunits) continue;
    bool coded = true;
    uint32_t pbyte = u;
    if (kCiera) {
      const uint32_t blk = (8u * u) >> p.log2B;
      coded = (s_bits[blk >> 5] >> (blk & 31u)) & 1u;
      pbyte = coded_before(u, s_bits, s_rank, p.log2B, p.nb, p.nch);
    }
    if (coded) {
      const uint32_t at = pbyte - p.sbase;
      const uint32_t p0 = s_planes[at];
      const uint32_t p1 = s_planes[kStage + at];
      const uint32_t p2 = s_planes[2u * kStage + at];
      const uint32_t vmask = kFull ? 0xFFu : ((min(8u, p.nc - 8u * u) == 8u) ? 0xFFu
                                                                           : ((1u << (p.nc - 8u * u)) - 1u));
      const uint2 codes = codes_from_planes(p0, p1, p2);
      ev[j] = make_uint2(exps_from_codes(codes.x, p.e0), exps_from_codes(codes.y, p.e0));
      const uint32_t em = ~(p0 | p1 | p2) & vmask;
      em4[j / 4u] |= em << (8u * (j % 4u));
      cnt[j] = __popc(em);
    }
  }
  const uint32_t pesc = part_escape_scan(cnt, base, s_tot);
  // Every escape read stays inside the chunk's escape section and the staged
  // bytes: the range's escapes must end inside both; the workgroup with the
  // part's last units checks the index entry after the part against before +
  // pesc, and the one with the chunk's last values checks the section's
  // padded length and the index entries of the quarters past the data.
  const uint32_t after = before + pesc;
  bool bad = after > p.esc_len || after - esc_lo > 16u * pieces;
  if (p.final_units && p.part + 1u < kParts) bad |= next != after;
  if (p.last_with_data) {
    bad |= pad128(after) != p.esc_len;
    for (uint32_t q = p.part + 1u; q < kParts; q++) bad |= (uint32_t(p.index >> (16u * q)) & 0xFFFFu) != after;
  }
  if (bad) return uint32_t(CIERA_ERR_FORMAT);  // uniform
#pragma unroll
  for (uint32_t j = 0; j < kU; j++) {
    const uint32_t u = p.u0 + j * kPartThreads + tid;
    if (!kFull && u >= p.nunits) continue;
    const uint32_t valid = kFull ? 8u : min(8u, p.nc - 8u * u);
    // the unit's escapes are staged bytes [before + base - esc_lo, + cnt)
    const uint32_t em = (em4[j / 4u] >> (8u * (j % 4u))) & 0xFFu;
    const uint2 e = merge_escapes(ev[j], em, s_esc, before + base[j] - esc_lo);
    store_unit(p.y, p.start + 8ull * u, valid, unit_join(smv[j], e));
    if (kCiera) {
      const uint32_t blk = (8u * u) >> p.log2B;
      if ((s_bits[blk >> 5] >> (blk & 31u)) & 1u) store_bytes8(p.cache + p.start + 8ull * u, valid, e);
    }
  }
  return 0u;
}

// Workgroup wg of one stream's decode: one part of a chunk (kS = 1), or one
// of its kS slices; workgroups never wait on each other, as the escape index
// gives each part its first escape.  It stores its status in *status.
template <bool kCiera, uint32_t kS>
__device__ __attribute__((always_inline)) inline void decode_workgroup(const uint8_t* __restrict__ in,
                                                                       uint64_t in_size, uint16_t* __restrict__ y,
                                                                       uint64_t n, uint64_t nchunks, uint32_t log2B,
                                                                       uint8_t* __restrict__ cache, uint32_t wg,
                                                                       uint32_t* __restrict__ status) {
  __shared__ __attribute__((aligned(16))) uint8_t s_planes[3u * kStage];
  __shared__ __attribute__((aligned(16))) uint8_t s_esc[kEscStage + 16u];
  __shared__ uint32_t s_ok;    // header and table entries are consistent
  __shared__ uint32_t s_fits;  // the chunk's fixed-size sections lie inside it
  __shared__ uint32_t s_e0;
  __shared__ uint64_t s_begin, s_end, s_index;
  __shared__ uint32_t s_bits[kBitmapWords];
  __shared__ uint32_t s_rank[kBitmapWords];
  __shared__ uint32_t s_tot[kUPT * kPartWaves + 1];
  const uint32_t tid = threadIdx.x;
  const uint32_t c = wg / (kParts * kS);
  const uint32_t h = (wg / kS) % kParts;
  const uint32_t slice = wg % kS;
  const uint32_t B = kCiera ? (1u << log2B) : 0u;
  const uint64_t base_off = table_end(nchunks);
  if (tid == 0) {
    uint32_t ok = 1u;
    const uint64_t* hd = reinterpret_cast<const uint64_t*>(in);
    const uint32_t magic = kCiera ? 0x52454943u : 0x3350495Au;
    uint64_t begin = 0, end = 0, index = 0;
    uint32_t e0 = 0;
    if (in_size < base_off) {
      ok = 0u;
    } else {
      // The table lies inside the stream once in_size >= base_off: its
      // entries are read with the header, in one round trip, and used only
      // if the header checks out.
      const uint64_t* table = reinterpret_cast<const uint64_t*>(in + kHeader);
      const uint64_t t_first = table[0], t_last = table[nchunks];
      if (nchunks) {
        begin = table[c];
        end = table[c + 1u];
        index = table[nchunks + 1u + c];
      }
      const uint64_t h0 = hd[0];
      e0 = uint32_t(h0 >> 56);
      ok &= uint32_t(h0 & 0xFFFFFFFFu) == magic;
      ok &= ((h0 >> 32) & 0xFFFFu) == 1u;
      ok &= ((h0 >> 48) & 0xFFu) == (kCiera ? 1u : 0u);
      ok &= e0 <= kMaxE0;
      ok &= hd[1] == n;
      ok &= hd[2] == (uint64_t(B) | (uint64_t(kChunk) << 32));
      ok &= hd[3] == nchunks;
      const uint64_t total = hd[4];
      ok &= total <= in_size;
      for (int i = 7; i < 16; i++) ok &= hd[i] == 0u;
      ok &= t_first == base_off;
      ok &= t_last == total;
      if (wg == 0u)  // the padding after the escape index is zero
        for (uint64_t i = 2u * nchunks + 1u; i < (base_off - kHeader) / 8u; i++) ok &= table[i] == 0u;
      if (nchunks) {
        ok &= begin >= base_off && begin <= end && end <= total;
        ok &= ((begin | end) & 127u) == 0u;
        ok &= (index & 0xFFFFu) == 0u;  // no escapes before the chunk's first value
      }
      if (!ok) begin = end = index = 0u;
    }
    s_ok = ok;
    s_e0 = e0;
    s_begin = begin;
    s_end = end;
    s_index = index;
  }
  __syncthreads();
  if (!s_ok || nchunks == 0u) {
    if (tid == 0) *status = s_ok ? 0u : uint32_t(CIERA_ERR_FORMAT);
    return;
  }
  const uint32_t e0 = s_e0;
  const uint64_t begin = s_begin, end = s_end;
  const uint64_t start = uint64_t(c) * kChunk;
  const uint32_t nc = uint32_t(min(uint64_t(kChunk), n - start));
  const uint32_t nunits = (nc + 7u) / 8u;
  const uint32_t pu0 = h * kPartUnits;

  uint32_t nch = 0, nb = 0;
  if (kCiera) {
    // the bitmap section must lie inside the chunk before it is read
    const uint64_t bm = begin + pad128(nc);
    const bool fits = bm + 128u <= end;
    nb = (nc + B - 1u) >> log2B;
    if (tid < 64u) {
      uint32_t w = 0;
      if (fits && tid < kBitmapWords) {
        w = *reinterpret_cast<const uint32_t*>(in + bm + 4u * tid);
        const uint32_t lo = 32u * tid;
        w = (lo >= nb) ? 0u : (nb - lo >= 32u ? w : (w & ((1u << (nb - lo)) - 1u)));
      }
      stage_bitmap(w, s_bits, s_rank);
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
    if (tid == 0) *status = uint32_t(CIERA_ERR_FORMAT);
    return;
  }
  constexpr uint32_t kRange = kPartUnits / kS;  // units of the workgroup
  const uint32_t u0 = pu0 + slice * kRange;
  if (u0 >= nunits) {  // a range past the chunk's data
    if (tid == 0) *status = 0u;
    return;
  }
  const uint32_t pb = uint32_t(g.plane_bytes);
  const uint32_t esc_len = uint32_t(end - g.esc);
  const uint64_t index = s_index;
  const uint32_t s_h = kCiera ? coded_before(pu0, s_bits, s_rank, log2B, nb, nch) : pu0;
  const uint32_t s_lo = kCiera ? coded_before(u0, s_bits, s_rank, log2B, nb, nch) : u0;
  const bool last_with_data = u0 + kRange >= nunits;
  // slots from the part's first unit to the end of the range (a block may
  // span several parts)
  const uint32_t s_next = kCiera ? coded_before(u0 + kRange, s_bits, s_rank, log2B, nb, nch)
                                 : min(u0 + kRange, nunits);
  DecodePart p;
  p.in = in;
  p.y = y;
  p.cache = cache;
  p.g = g;
  p.start = start;
  p.nc = nc;
  p.nunits = nunits;
  p.pu0 = pu0;
  p.e0 = e0;
  p.pb = pb;
  p.esc_len = esc_len;
  p.sbase = s_h;  // a multiple of 8 for a part holding values
  p.stage_len = (s_next + 7u) / 8u * 8u - s_h;  // <= kPartUnits + 8
  p.last_with_data = last_with_data;
  p.log2B = log2B;
  p.nb = nb;
  p.nch = nch;
  p.part = h;
  p.index = index;
  p.before = uint32_t(index >> (16u * h)) & 0xFFFFu;
  p.u0 = u0;
  p.slot0 = s_lo;
  p.final_units = slice + 1u == kS || last_with_data;
  uint32_t err;
  if (8u * (u0 + kRange) <= nc)
    err = decode_part<kCiera, true, kS>(p, s_bits, s_rank, s_planes, s_esc, s_tot);
  else
    err = decode_part<kCiera, false, kS>(p, s_bits, s_rank, s_planes, s_esc, s_tot);
  if (tid == 0) *status = err;
}

// One stream: workgroup b decodes its piece b.
template <bool kCiera, uint32_t kS>
__global__ __launch_bounds__(kPartThreads) void k_decode(const uint8_t* __restrict__ in, uint64_t in_size,
                                                         uint16_t* __restrict__ y, uint64_t n, uint64_t nchunks,
                                                         uint32_t log2B, uint8_t* __restrict__ cache,
                                                         uint64_t* __restrict__ n_err_slots,
                                                         uint32_t* __restrict__ err_slots) {
  if (blockIdx.x == 0u && threadIdx.x == 0u) *n_err_slots = gridDim.x;
  decode_workgroup<kCiera, kS>(in, in_size, y, n, nchunks, log2B, cache, blockIdx.x, err_slots + blockIdx.x);
}

// Several streams of the same n and B in one launch (a rank's received peer
// shards): workgroup b decodes piece b % per of stream b / per, with that
// stream's input, output and receiver cache, and status word b.
struct DecodeStreams {
  const uint8_t* in[kDecodeBatchMax];
  uint64_t in_size[kDecodeBatchMax];
  uint16_t* y[kDecodeBatchMax];
  uint8_t* cache[kDecodeBatchMax];
};
template <bool kCiera, uint32_t kS>
__global__ __launch_bounds__(kPartThreads) void k_decode_batch(DecodeStreams st, uint32_t per, uint64_t n,
                                                               uint64_t nchunks, uint32_t log2B,
                                                               uint64_t* __restrict__ n_err_slots,
                                                               uint32_t* __restrict__ err_slots) {
  const uint32_t i = blockIdx.x / per;  // uniform: the workgroup's stream
  if (blockIdx.x == 0u && threadIdx.x == 0u) *n_err_slots = gridDim.x;
  decode_workgroup<kCiera, kS>(st.in[i], st.in_size[i], st.y[i], n, nchunks, log2B, st.cache[i], blockIdx.x - i * per,
                               err_slots + blockIdx.x);
}

// ------------------------------------------------------------------ rANS modes
// The coded exponents (all of them in zip3 mode, those of changed blocks in
// ciera mode) entropy coded with range ANS in place of the 3-bit code, as the
// CIERA page ANS-codes changed exponents (section 3.1); the page names no ANS
// parameters, so the coder is our own:
//  - symbols: a chunk's coded exponents; part h of the chunk (its values
//    16384 h .. 16384 h + 16383) codes its own ones in value order;
//  - one frequency table per chunk: the histogram of all its coded
//    exponents normalised to M = 4096 (with d distinct symbols among m,
//    f = max(1, floor(h (M - d) / m)) for each present symbol, the rest to
//    the most frequent one, the lowest on ties);
//  - per part, 64 interleaved 32-bit states (symbol i of the part to state
//    i mod 64) in [2^16, 2^32), starting at 2^16; encode: if x >= f 2^20
//    emit its low 16 bits and shift, then x = (x div f) M + x mod f + c;
//    decode: slot = x mod M, x = f (x div M) + slot - c, then one 16-bit
//    word if x < 2^16;
//  - chunk payload: u8 lo, u8 hi, u16 0, u16 w_0 .. w_3 (the words of each
//    part's stream, 0 without coded symbols), u16 f_lo .. f_hi, then the
//    part streams in part order: the 64 final states (low, high half), then
//    the words each step emitted, steps in decode order, states ascending
//    within a step;
//  - stream (version 2): header (mode 2 zip3 + rANS, 3 ciera + rANS; bytes
//    48..55 the coded symbols), a table of nchunks + 1 u64 chunk payload
//    offsets, every value's sign+mantissa byte, in ciera mode 128 bitmap
//    bytes per chunk, then the chunk payloads, each padded to 128 bytes.
// One workgroup per chunk; wave h codes part h against the chunk's table in
// LDS, so the four serial coders of a chunk run at once.  Encode: k_stats
// (per part, the histogram of its coded exponents), k_rans_enc (code the
// parts into the chunk's scratch slot, find the offset by look-back over the
// chunks before, copy into the stream), k_rans_finish (header totals).
// Decode: k_rans_dec.
constexpr uint32_t kRansM = 4096u;
constexpr uint32_t kRansL = 1u << 16;
constexpr uint32_t kRansStates = 64u;
constexpr uint32_t kRansVersion = 2u;
constexpr uint32_t kRansHead = 12u;                                 // payload bytes before the table
constexpr uint32_t kRansPartWords = 2u * kRansStates + kPartValues;  // a part stream's largest word count
constexpr uint32_t kRansSlot = kParts * 2u * kRansPartWords;         // scratch per chunk: one region per part
constexpr uint32_t kRansBlock = 1024u;   // payload bytes per block of a decoding wave's LDS ring
constexpr uint32_t kRansWin = 8u;        // steps whose inputs a coding wave loads ahead
constexpr uint32_t kSpanUnits = 8u;      // units of unchanged blocks a decoding thread moves at a time (ciera)
constexpr uint32_t kGranules = kPartValues / 64u;  // a part's largest granule count (B = 64)

__host__ __device__ inline uint64_t rans_sm_pos(uint64_t nchunks) { return kHeader + pad128(8u * (nchunks + 1u)); }
__host__ __device__ inline uint64_t rans_pay_pos(uint64_t n, uint64_t nchunks, bool ciera) {
  return rans_sm_pos(nchunks) + pad128(n) + (ciera ? 128u * nchunks : 0u);
}
// Largest payload of a chunk of nc values: every value coded, at most one
// word per symbol.
__host__ __device__ inline uint64_t rans_chunk_max(uint64_t nc) {
  return nc ? kRansHead + 2u * kBins + 2u * (2u * kRansStates * cdiv(nc, kPartValues) + nc) : 0u;
}

// The coded values of part h (wave h).  Its values fall into granules of
// G = min(B, 16384) values (zip3: one granule, always coded); granule j of
// the chunk (j = h 16384 / G + g) is coded when its block changed and it
// holds values.  Their chunk-relative indices go to gl in order, so that
// symbol i of the part is value gl[i >> log2G] G + (i mod G) of the chunk.
// Returns the part's coded values (every lane of the wave).
__device__ inline uint32_t part_granules(uint32_t h, uint32_t nc, uint32_t log2B, uint32_t log2G, bool ciera,
                                         const uint32_t* s_bits, uint16_t* gl) {
  const uint32_t lane = lane_id();
  const uint32_t G = 1u << log2G, ng = kPartValues >> log2G;
  const uint64_t below = (1ull << lane) - 1u;
  uint32_t nl = 0, m = 0;
  for (uint32_t g0 = 0; g0 < ng; g0 += 64u) {
    const uint32_t g = g0 + lane;
    const uint32_t j = h * ng + g;
    uint32_t cnt = 0;
    if (g < ng && j * G < nc) {
      cnt = min(G, nc - j * G);
      if (ciera) {
        const uint32_t blk = j >> (log2B - log2G);
        if (!((s_bits[blk >> 5] >> (blk & 31u)) & 1u)) cnt = 0;
      }
    }
    const uint64_t mk = __ballot(cnt != 0u);
    if (cnt) gl[nl + uint32_t(__popcll(mk & below))] = uint16_t(j);
    nl += uint32_t(__popcll(mk));
    m += cnt;
  }
  return wave_sum_u32(m);
}

// The block's ready flag and inclusive prefix or own size, as in the
// single-read encode: kFlagSize | padded payload bytes, then kFlagIncl |
// payload bytes of the parts up to and including it.
__device__ inline bool part_lookback(const uint64_t* rstat, uint64_t p, uint64_t& before, uint32_t limit) {
  const uint32_t lane = lane_id();
  before = 0;
  int64_t top = int64_t(p) - 1;
  uint32_t spins = 0;
  while (top >= 0) {
    const int64_t k = top - int64_t(lane);
    const uint64_t st = (k >= 0) ? load_relaxed(&rstat[uint64_t(k) * kRstatStride]) : kFlagIncl;
    const uint64_t flag = st & ~kValMask;
    if (__ballot(flag == 0u) != 0u) {
      if (++spins > limit) return false;
      __builtin_amdgcn_s_sleep(1);
      continue;
    }
    const uint64_t incl = __ballot(flag == kFlagIncl);
    if (incl != 0u) {
      const uint32_t first = uint32_t(__builtin_ctzll(incl));
      before += wave_sum_u64(lane <= first ? (st & kValMask) : 0u);
      return true;
    }
    before += wave_sum_u64(st & kValMask);
    top -= 64;
  }
  return true;
}

// Encoder table entry of a symbol with frequency f >= 1 and cumulative
// frequency c: x = thr is the largest state that needs no renormalisation
// word (f 2^20 - 1), rfd a FP32 value a little below 1 / f, nf = -f, and
// c | f << 16.
struct RansEnt {
  uint32_t thr;
  float rfd;
  int32_t nf;
  uint32_t cf;
};
__device__ inline RansEnt rans_entry(uint32_t f, uint32_t c) {
  RansEnt e;
  e.thr = uint32_t((uint64_t(f) << 20) - 1u);
  // rounded down from (1 - 2^-22) / f, so rfd (1 + 2^-24)^2 < 1 / f and
  // rfd > (1 - 2^-21) / f
  e.rfd = __double2float_rd((1.0 - 0x1p-22) / double(f));
  e.nf = -int32_t(f);
  e.cf = c | (f << 16);
  return e;
}

// One encoder state update, x = (x div f) M + (x mod f) + c, for
// x < f 2^20 (the state after its renormalisation).  x and the product with
// rfd are each rounded to FP32 (relative error 2^-24 each), so the product
// p lies in ((1 - 2^-21) x / f, x / f]; as x / f < 2^20, p > x / f - 1/2.
// Its truncation q0 is thus the quotient Q or Q - 1, and r0 = x - q0 f, exact
// in 32 bits, is below 2 f: Q = q0 + (r0 >= f).  Then
// x (div f) M + x mod f + c = x + c + Q (M - f) = (Q << 12) + x + c - Q f.
__device__ inline uint32_t rans_push(uint32_t x, const RansEnt& e) {
  const uint32_t q0 = uint32_t(float(x) * e.rfd);                     // < 2^20: 24-bit products suffice
  const uint32_t r0 = uint32_t(__mul24(int32_t(q0), e.nf) + int32_t(x));  // exact: 0 <= r0 < 2 f
  const uint32_t q = q0 + ((r0 >= (e.cf >> 16)) ? 1u : 0u);
  return uint32_t(__mul24(int32_t(q), e.nf)) + ((q << 12) + x + (e.cf & 0xFFFFu));
}


template <bool kCiera>
__global__ __launch_bounds__(kPartThreads) void k_rans_enc(const uint16_t* __restrict__ x, uint64_t n,
                                                           uint64_t nchunks, uint32_t log2B,
                                                           uint8_t* __restrict__ out, Ws ws) {
  __shared__ uint32_t s_f[kBins];
  __shared__ RansEnt s_ent[kBins];
  __shared__ uint16_t s_gl[kParts][kGranules];
  __shared__ __attribute__((aligned(16))) uint8_t s_sym[kPartWaves][kRansWin * kRansStates];
  __shared__ uint32_t s_bits[kBitmapWords], s_rank[kBitmapWords];
  __shared__ uint32_t s_w[kPartWaves];
  __shared__ uint32_t s_m[kParts], s_nw[kParts], s_wpos[kParts];
  __shared__ uint32_t s_lohi, s_ok;
  __shared__ uint64_t s_before;
  __shared__ uint32_t s_found;
  const uint32_t tid = threadIdx.x, lane = lane_id();
  const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: per-wave addresses stay scalar
  const uint64_t c = blockIdx.x;
  const uint32_t B = kCiera ? (1u << log2B) : 0u;
  const uint32_t log2G = kCiera ? min(log2B, 14u) : 14u;
  const uint64_t start = c * kChunk;
  const uint32_t nc = uint32_t(min(uint64_t(kChunk), n - start));
  const uint64_t sm_pos = rans_sm_pos(nchunks);

  if (kCiera && tid < 64u)
    stage_bitmap((tid < kBitmapWords) ? chunk_bitmap_word(ws.bitmap + c * kBitmapWords, tid, B) : 0u, s_bits,
                 s_rank);
  __syncthreads();
  const uint32_t mh = part_granules(wave, nc, log2B, log2G, kCiera, s_bits, s_gl[wave]);
  if (lane == 0u) s_m[wave] = mh;
  if (kCiera) {
    // sign+mantissa bytes of the values that are not coded (the coders write
    // those of the coded ones)
    const uint32_t nunits = (nc + 7u) / 8u;
    for (uint32_t u = tid; u < nunits; u += kPartThreads) {
      const uint32_t blk = (8u * u) >> log2B;
      if ((s_bits[blk >> 5] >> (blk & 31u)) & 1u) continue;
      const uint32_t k = min(8u, nc - 8u * u);
      store_bytes8(out + sm_pos + start + 8ull * u, k, unit_sm(load_unit(x, start + 8ull * u, k)));
    }
  }
  __syncthreads();
  const uint32_t m = s_m[0] + s_m[1] + s_m[2] + s_m[3];

  // frequencies from the parts' histogram rows (one symbol per thread); a
  // part without coded values adds nothing (with B > 16384 its row counts
  // all of its values, which its unchanged block leaves uncoded)
  uint32_t hs = 0;
#pragma unroll
  for (uint32_t h = 0; h < kParts; h++)
    if (s_m[h]) hs += ws.hist[(c * kParts + h) * kBins + tid];
  const uint32_t hsum = part_sum_u32(hs, s_w);
  const uint32_t d = part_sum_u32(hs ? 1u : 0u, s_w);
  // most frequent symbol, the lowest on ties: max of (h << 8) | (255 - s)
  uint32_t key = (hs << 8) | (255u - tid);
  for (uint32_t o = 32; o >= 1; o >>= 1) key = max(key, uint32_t(__shfl_xor(int(key), int(o))));
  __syncthreads();
  if (lane == 0u) s_w[wave] = key;
  __syncthreads();
  key = max(max(s_w[0], s_w[1]), max(s_w[2], s_w[3]));
  const uint32_t top = 255u - (key & 0xFFu);
  uint32_t f = 0;
  if (hs) {
    f = uint32_t(uint64_t(hs) * (kRansM - d) / max(hsum, 1u));
    if (f == 0u) f = 1u;
  }
  const uint32_t fsum = part_sum_u32(f, s_w);
  if (tid == top) f += kRansM - fsum;
  const uint32_t cum_incl = part_incl_scan_u32(f, s_w);
  s_f[tid] = f;
  s_ent[tid] = rans_entry(max(f, 1u), cum_incl - f);  // (symbols with f = 0 are never coded)
  // first and last symbol with f > 0
  uint32_t lo = f ? tid : 255u, hi = f ? tid : 0u;
  for (uint32_t o = 32; o >= 1; o >>= 1) {
    lo = min(lo, uint32_t(__shfl_xor(int(lo), int(o))));
    hi = max(hi, uint32_t(__shfl_xor(int(hi), int(o))));
  }
  __syncthreads();
  if (lane == 0u) s_w[wave] = lo | (hi << 16);
  __syncthreads();
  if (tid == 0) {
    uint32_t l = 255u, u = 0u;
    for (uint32_t w = 0; w < kPartWaves; w++) {
      l = min(l, s_w[w] & 0xFFFFu);
      u = max(u, s_w[w] >> 16);
    }
    s_lohi = l | (u << 8);
    s_ok = (hsum == m) ? 1u : 0u;  // the histograms counted exactly the coded values
  }
  __syncthreads();
  const bool ok = s_ok != 0u;

  // Wave h codes part h, last step first, into its region of the chunk's
  // scratch slot from the region's end.  It takes its symbols in groups of
  // kRansWin steps (512 symbols): lane l loads the 8 values of symbols
  // 512 g + 8 l .. + 7 (one 16-byte load, contiguous through the granule
  // list), writes their sign+mantissa bytes (one 8-byte store) and stages
  // their exponents in the wave's LDS buffer, from which each step reads its
  // symbol.  A group's loads are issued while the group above it codes (two
  // buffers take turns); the top group, the only one that can be partial,
  // goes first on its own.
  uint16_t* reg = reinterpret_cast<uint16_t*>(ws.rslot + c * uint64_t(kRansSlot)) + wave * kRansPartWords;
  uint32_t wpos = kRansPartWords;
  if (mh && ok) {
    const uint16_t* gl = s_gl[wave];
    uint8_t* sym = s_sym[wave];
    const uint32_t gmask = (1u << log2G) - 1u;
    constexpr uint32_t kGroup = kRansWin * kRansStates;
    auto value_of = [&](uint32_t i) -> uint32_t {  // chunk-relative value of the part's symbol i
      return kCiera ? ((uint32_t(gl[i >> log2G]) << log2G) | (i & gmask)) : (wave * kPartValues + i);
    };
    uint32_t xs = kRansL;
    uint8_t* reg8 = reinterpret_cast<uint8_t*>(reg);
    auto code = [&](uint32_t t, const RansEnt& e, bool full) {
      const bool act = full || t * kRansStates + lane < mh;
      const bool emit = act && xs > e.thr;  // x >= f 2^20
      const uint64_t mk = __ballot(emit);
      const uint32_t ne = uint32_t(__popcll(mk));
      const uint32_t rank = __builtin_amdgcn_mbcnt_hi(uint32_t(mk >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(mk), 0u));
      // (a 32-bit byte offset from the wave's base: one address operand)
      wpos = __builtin_amdgcn_readfirstlane(wpos - ne);  // uniform: keep it scalar
      if (emit) *reinterpret_cast<uint16_t*>(reg8 + 2u * (wpos + rank)) = uint16_t(xs & 0xFFFFu);
      xs >>= emit ? 16u : 0u;
      const uint32_t xn = rans_push(xs, e);
      xs = act ? xn : xs;
    };
    // one group: the lane's sign+mantissa bytes out, its exponents staged,
    // then the group's steps from the highest
    auto group = [&](uint32_t g, const Unit& u, uint32_t vi, uint32_t cnt, bool full) {
      store_bytes8(out + sm_pos + start + vi, cnt, unit_sm(u));
      *reinterpret_cast<uint2*>(sym + 8u * lane) = unit_exponents(u);
      __builtin_amdgcn_wave_barrier();
      // the steps' table entries, read before the state chain needs them
      RansEnt ev[kRansWin];
#pragma unroll
      for (uint32_t k = 0; k < kRansWin; k++) ev[k] = s_ent[sym[k * kRansStates + lane]];
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int32_t k = int32_t(kRansWin) - 1; k >= 0; k--) {
        const uint32_t t = g * kRansWin + uint32_t(k);
        if (full || t * kRansStates < mh) code(t, ev[k], full);
      }
    };
    const uint32_t ng = cdiv(mh, kGroup);
    {
      const uint32_t i0 = (ng - 1u) * kGroup + 8u * lane;
      const uint32_t cnt = (i0 < mh) ? min(8u, mh - i0) : 0u;
      const uint32_t vi = value_of(cnt ? i0 : 0u);
      Unit u;
      u.w[0] = u.w[1] = u.w[2] = u.w[3] = 0u;
      if (cnt) u = load_unit(x, start + vi, cnt);
      group(ng - 1u, u, vi, cnt, false);
    }
    if (ng >= 2u) {
      // full groups: every lane has 8 values, so every load is issued
      auto fetch = [&](uint32_t g, Unit& u, uint32_t& vi) {
        vi = value_of(g * kGroup + 8u * lane);
        const uint4 v = *reinterpret_cast<const uint4*>(x + start + vi);
        u.w[0] = v.x;
        u.w[1] = v.y;
        u.w[2] = v.z;
        u.w[3] = v.w;
      };
      Unit ua, ub;
      uint32_t va, vb;
      uint32_t g = ng - 2u;
      fetch(g, ua, va);
      while (true) {
        fetch(g ? g - 1u : 0u, ub, vb);
        group(g, ua, va, 8u, true);
        if (g-- == 0u) break;
        fetch(g ? g - 1u : 0u, ua, va);
        group(g, ub, vb, 8u, true);
        if (g-- == 0u) break;
      }
    }
    wpos -= 2u * kRansStates;
    reg[wpos + 2u * lane] = uint16_t(xs & 0xFFFFu);
    reg[wpos + 2u * lane + 1u] = uint16_t(xs >> 16);
  }
  if (lane == 0u) {
    s_nw[wave] = kRansPartWords - wpos;
    s_wpos[wave] = wpos;
  }
  __syncthreads();
  const uint32_t lo_s = s_lohi & 0xFFu, hi_s = s_lohi >> 8;
  const uint32_t span = hi_s - lo_s + 1u;
  const uint32_t w0 = s_nw[0], w1 = s_nw[1], w2 = s_nw[2], w3 = s_nw[3];
  const uint32_t words = w0 + w1 + w2 + w3;
  const uint64_t bytes = (m && ok) ? kRansHead + 2u * span + 2u * uint64_t(words) : 0u;
  const uint64_t padded = pad128(bytes);

  // offset: publish the padded size, look back over the chunks before
  if (tid == 0) store_relaxed(&ws.rstat[c * kRstatStride], kFlagSize | padded);
  if (wave == 0) {
    uint64_t before = 0;
    const bool found = part_lookback(ws.rstat, c, before, ws.spin_limit);
    if (lane == 0) {
      s_before = before;
      s_found = found ? 1u : 0u;
      if (found) store_relaxed(&ws.rstat[c * kRstatStride], kFlagIncl | (before + padded));
    }
  }
  __syncthreads();
  const uint32_t err = (!ok || !s_found) ? uint32_t(CIERA_ERR_INTERNAL) : 0u;
  if (tid == 0) ws.err[c] = err;
  if (err) return;
  const uint64_t at = rans_pay_pos(n, nchunks, kCiera) + s_before;
  uint64_t* table = reinterpret_cast<uint64_t*>(out + kHeader);
  if (tid == 0) {
    table[c] = at;
    ws.rinfo[c] = uint64_t(m) |
                  (uint64_t(kCiera ? s_rank[kBitmapWords - 1] + __popc(s_bits[kBitmapWords - 1]) : 0u) << 32);
    if (c + 1u == nchunks) table[nchunks] = at + padded;
  }
  if (bytes) {
    // head, table, then the part streams (u16 aligned: the payload starts on
    // 128 bytes and its head and table take an even number of bytes)
    uint16_t* dst = reinterpret_cast<uint16_t*>(out + at);
    if (tid < 6u) {
      const uint32_t v = (tid == 0) ? (lo_s | (hi_s << 8)) : (tid == 1) ? 0u : s_nw[tid - 2u];
      dst[tid] = uint16_t(v);
    }
    for (uint32_t k = tid; k < span; k += kPartThreads) dst[kRansHead / 2u + k] = uint16_t(s_f[lo_s + k]);
    // The part streams, from their regions of the scratch slot (16-byte
    // aligned) to their place after the table (any even offset), the blocks
    // of all four parts dealt to the threads in one pass: a thread builds
    // one 16-byte block of the payload from the two aligned source blocks
    // that cover it (a source block outside the part's region holds no byte
    // of the part and is not read) and stores it whole, or, for a part's
    // first and last blocks, which it shares with what comes before and
    // after, as the u16 units that belong to the part.
    const uint8_t* __restrict__ slot = ws.rslot + c * uint64_t(kRansSlot);
    uint8_t* __restrict__ pay = out + at;
    uint32_t dp[kParts], ln[kParts], cum[kParts + 1];
    int32_t dl[kParts];
    cum[0] = 0u;
    uint32_t dpos = kRansHead + 2u * span;  // a part's first byte in the payload
#pragma unroll
    for (uint32_t h = 0; h < kParts; h++) {
      dp[h] = dpos;
      ln[h] = 2u * s_nw[h];
      dl[h] = int32_t(h * 2u * kRansPartWords + 2u * s_wpos[h]) - int32_t(dpos);  // source byte = payload byte + dl
      cum[h + 1] = cum[h] + (ln[h] ? (dpos + ln[h] - 1u) / 16u - dpos / 16u + 1u : 0u);
      dpos += ln[h];
    }
    for (uint32_t k = tid; k < cum[kParts]; k += kPartThreads) {
      uint32_t h = 0, d_lo = dp[0], d_len = ln[0], kb = cum[0];
      int32_t delta = dl[0];
#pragma unroll
      for (uint32_t j = 1; j < kParts; j++)
        if (k >= cum[j]) { h = j; d_lo = dp[j]; d_len = ln[j]; delta = dl[j]; kb = cum[j]; }
      const int32_t region = int32_t(h * 2u * kRansPartWords), region_end = region + int32_t(2u * kRansPartWords);
      const uint32_t b_first = d_lo / 16u, b_last = (d_lo + d_len - 1u) / 16u, b = b_first + (k - kb);
      const uint32_t d0 = 16u * b;
      const int32_t a0 = (int32_t(d0) + delta) & ~15;
      const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
      const uint4 p = (a0 >= region) ? *reinterpret_cast<const uint4*>(slot + a0) : zero;
      const uint4 q = (a0 + 16 < region_end) ? *reinterpret_cast<const uint4*>(slot + a0 + 16) : zero;
      const uint4 v = shift_bytes(p, q, uint32_t(delta) & 15u);
      if (b != b_first && b != b_last) {
        *reinterpret_cast<uint4*>(pay + d0) = v;
      } else {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (uint32_t i = 0; i < 8u; i++) {
          const uint32_t di = d0 + 2u * i;
          if (di >= d_lo && di < d_lo + d_len)
            *reinterpret_cast<uint16_t*>(pay + di) = uint16_t(w[i / 2u] >> (16u * (i % 2u)));
        }
      }
    }
    for (uint64_t k = bytes + tid; k < padded; k += kPartThreads) out[at + k] = 0u;
  }
  // the chunk's bitmap
  if (kCiera && tid < kBitmapWords)
    *reinterpret_cast<uint32_t*>(out + sm_pos + pad128(n) + 128u * c + 4u * tid) = s_bits[tid];
}

// Header and the chunk table's padding; the totals of coded symbols and
// changed blocks from the chunks' records.  One workgroup.
__global__ __launch_bounds__(kThreads) void k_rans_finish(uint64_t n, uint64_t nchunks, uint32_t B,
                                                          uint8_t* __restrict__ out, uint64_t* __restrict__ out_size,
                                                          Ws ws) {
  __shared__ uint64_t s_m[kThreads / 64u], s_c[kThreads / 64u];
  const uint32_t tid = threadIdx.x;
  uint64_t* hd = reinterpret_cast<uint64_t*>(out);
  uint64_t* table = reinterpret_cast<uint64_t*>(out + kHeader);
  if (tid == 0) ws.ctrl->n_err_slots = nchunks;
  uint64_t m = 0, ch = 0;
  for (uint64_t i = tid; i < nchunks; i += kThreads) {
    const uint64_t r = ws.rinfo[i];
    m += r & 0xFFFFFFFFu;
    ch += r >> 32;
  }
  m = wave_sum_u64(m);
  ch = wave_sum_u64(ch);
  if (lane_id() == 0u) {
    s_m[tid >> 6] = m;
    s_c[tid >> 6] = ch;
  }
  const uint64_t sm_pos = rans_sm_pos(nchunks);
  for (uint64_t i = nchunks + 1u + tid; i < (sm_pos - kHeader) / 8u; i += kThreads) table[i] = 0u;
  __syncthreads();
  if (tid == 0) {
    uint64_t tm = 0, tc = 0;
    for (uint32_t w = 0; w < kThreads / 64u; w++) {
      tm += s_m[w];
      tc += s_c[w];
    }
    const bool ciera = B != 0u;
    if (nchunks == 0u) table[0] = rans_pay_pos(n, nchunks, ciera);
    const uint64_t total = table[nchunks];
    const uint32_t magic = ciera ? 0x52454943u /* "CIER" */ : 0x3350495Au /* "ZIP3" */;
    hd[0] = uint64_t(magic) | (uint64_t(kRansVersion) << 32) | (uint64_t(ciera ? 3u : 2u) << 48);
    hd[1] = n;
    hd[2] = uint64_t(B) | (uint64_t(kChunk) << 32);
    hd[3] = nchunks;
    hd[4] = total;
    hd[5] = tc;
    hd[6] = tm;
    for (int i = 7; i < 16; i++) hd[i] = 0u;
    *out_size = total;
    // zero padding after the sign+mantissa bytes
    for (uint64_t i = sm_pos + n; i < sm_pos + pad128(n); i++) out[i] = 0u;
  }
}

template <bool kCiera>
__global__ __launch_bounds__(kPartThreads) void k_rans_dec(const uint8_t* __restrict__ in, uint64_t in_size,
                                                           uint16_t* __restrict__ y, uint64_t n, uint64_t nchunks,
                                                           uint32_t log2B, uint8_t* __restrict__ cache,
                                                           uint64_t* __restrict__ n_err_slots,
                                                           uint32_t* __restrict__ err_slots) {
  // per wave, a ring of 4 payload blocks of 1 KB (block j in slot j mod 4)
  __shared__ __attribute__((aligned(16))) uint8_t s_ring[kPartWaves][4u * kRansBlock];
  // per slot: symbol | (f - 1) << 8 | (slot - cum) << 20
  __shared__ uint32_t s_dtab[kRansM];
  // f and cum per symbol while the slot table is built, then the waves'
  // decoded-symbol buffers (kRansWin steps each)
  __shared__ __attribute__((aligned(16))) uint32_t s_fcum[2u * kBins];
  static_assert(2u * kBins * 4u >= kPartWaves * kRansWin * kRansStates, "symbol buffers fit");
  uint32_t* s_f = s_fcum;
  uint32_t* s_cum = s_fcum + kBins;
  uint8_t* s_sym = reinterpret_cast<uint8_t*>(s_fcum);
  __shared__ uint16_t s_gl[kParts][kGranules];
  __shared__ uint32_t s_bits[kBitmapWords], s_rank[kBitmapWords];
  __shared__ uint32_t s_w[kPartWaves];
  __shared__ uint32_t s_m[kParts], s_nw[kParts];
  __shared__ uint32_t s_ok;
  __shared__ uint64_t s_a, s_b;
  const uint32_t tid = threadIdx.x, lane = lane_id();
  const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: per-wave addresses stay scalar
  const uint64_t c = blockIdx.x;
  const uint32_t B = kCiera ? (1u << log2B) : 0u;
  const uint32_t log2G = kCiera ? min(log2B, 14u) : 14u;
  const uint64_t sm_pos = rans_sm_pos(nchunks);
  const uint64_t bm_pos = sm_pos + pad128(n);
  const uint64_t pay_pos = rans_pay_pos(n, nchunks, kCiera);
  if (tid == 0) {
    uint32_t ok = 1u;
    uint64_t a = 0, b = 0;
    const uint64_t* hd = reinterpret_cast<const uint64_t*>(in);
    if (in_size < pay_pos) {
      ok = 0u;
    } else {
      const uint32_t magic = kCiera ? 0x52454943u : 0x3350495Au;
      ok &= hd[0] == (uint64_t(magic) | (uint64_t(kRansVersion) << 32) | (uint64_t(kCiera ? 3u : 2u) << 48));
      ok &= hd[1] == n;
      ok &= hd[2] == (uint64_t(B) | (uint64_t(kChunk) << 32));
      ok &= hd[3] == nchunks;
      // in_size is the buffer's size: the stream's own length may be less
      const uint64_t total = hd[4];
      ok &= total <= in_size;
      for (int i = 7; i < 16; i++) ok &= hd[i] == 0u;
      const uint64_t* table = reinterpret_cast<const uint64_t*>(in + kHeader);
      ok &= table[0] == pay_pos && table[nchunks] == total;
      if (ok && nchunks > 0u) {
        a = table[c];
        b = table[c + 1u];
        ok &= a >= pay_pos && a <= b && b <= total && ((a | b) & 127u) == 0u;
      }
    }
    s_ok = ok;
    s_a = a;
    s_b = b;
    if (c == 0u) *n_err_slots = gridDim.x;
  }
  __syncthreads();
  if (!s_ok || nchunks == 0u) {  // an empty tensor: the header and table are all there is
    if (tid == 0) err_slots[c] = s_ok ? 0u : uint32_t(CIERA_ERR_FORMAT);
    return;
  }
  const uint64_t a = s_a, b = s_b;
  const uint64_t start = c * kChunk;
  const uint32_t nc = uint32_t(min(uint64_t(kChunk), n - start));
  bool bad = false;
  if (kCiera && tid < 64u) {
    const uint32_t w = (tid < kBitmapWords) ? *reinterpret_cast<const uint32_t*>(in + bm_pos + 128u * c + 4u * tid) : 0u;
    // no bit past the chunk's last block
    const uint32_t nb = (nc + B - 1u) >> log2B;
    const uint32_t lo_bit = 32u * tid;
    const uint32_t valid = (lo_bit >= nb) ? 0u : ((nb - lo_bit >= 32u) ? ~0u : ((1u << (nb - lo_bit)) - 1u));
    if (w & ~valid) bad = true;
    stage_bitmap(w & valid, s_bits, s_rank);
  }
  __syncthreads();
  const uint32_t mh = part_granules(wave, nc, log2B, log2G, kCiera, s_bits, s_gl[wave]);
  if (lane == 0u) s_m[wave] = mh;
  if (kCiera) {
    // values of unchanged blocks: sign+mantissa byte and the receiver cache,
    // kSpanUnits units per thread at a time with all their loads issued
    // before the first store
    const uint32_t nunits = (nc + 7u) / 8u;
    for (uint32_t u0 = 0; u0 < nunits; u0 += kSpanUnits * kPartThreads) {
      uint2 smv[kSpanUnits], ev[kSpanUnits];
      uint32_t keep = 0;
      if (8u * (u0 + kSpanUnits * kPartThreads) <= nc) {
        // Every unit of the span holds 8 values.  No load sits under a
        // per-lane condition (the compiler would copy its result into place
        // after a wait for all loads before it): from B = 512 on, a wave's 64
        // units lie in one block, so the wave loads them or skips them
        // together; below, a unit of a changed block reads the chunk's first
        // bytes instead.  Units of changed blocks are not stored.
        if (log2B >= 9u) {
#pragma unroll
          for (uint32_t j = 0; j < kSpanUnits; j++) {
            const uint32_t u = u0 + j * kPartThreads + tid;
            const uint32_t blk = (8u * u) >> log2B;
            const bool kept = !((s_bits[blk >> 5] >> (blk & 31u)) & 1u);
            // any value where the wave skips: none of its units is stored
            uint64_t sv = __builtin_nondeterministic_value(sv), cv = __builtin_nondeterministic_value(cv);
            if (__ballot(kept) != 0u) {
              sv = *reinterpret_cast<const uint64_t*>(in + sm_pos + start + 8ull * u);
              cv = *reinterpret_cast<const uint64_t*>(cache + start + 8ull * u);
            }
            smv[j] = make_uint2(uint32_t(sv), uint32_t(sv >> 32));
            ev[j] = make_uint2(uint32_t(cv), uint32_t(cv >> 32));
            keep |= uint32_t(kept) << j;
          }
        } else {
#pragma unroll
          for (uint32_t j = 0; j < kSpanUnits; j++) {
            const uint32_t u = u0 + j * kPartThreads + tid;
            const uint32_t blk = (8u * u) >> log2B;
            const bool kept = !((s_bits[blk >> 5] >> (blk & 31u)) & 1u);
            const uint64_t off = kept ? 8ull * u : 0ull;
            smv[j] = *reinterpret_cast<const uint2*>(in + sm_pos + start + off);
            ev[j] = *reinterpret_cast<const uint2*>(cache + start + off);
            keep |= uint32_t(kept) << j;
          }
        }
      } else {
#pragma unroll
        for (uint32_t j = 0; j < kSpanUnits; j++) {
          const uint32_t u = u0 + j * kPartThreads + tid;
          const uint32_t blk = (8u * u) >> log2B;
          smv[j] = ev[j] = make_uint2(0u, 0u);
          if (u < nunits && !((s_bits[blk >> 5] >> (blk & 31u)) & 1u)) {
            const uint32_t k = min(8u, nc - 8u * u);
            smv[j] = load_bytes8(in + sm_pos + start + 8ull * u, k);
            ev[j] = load_bytes8(cache + start + 8ull * u, k);
            keep |= 1u << j;
          }
        }
      }
#pragma unroll
      for (uint32_t j = 0; j < kSpanUnits; j++) {
        const uint32_t u = u0 + j * kPartThreads + tid;
        if ((keep >> j) & 1u) store_unit(y, start + 8ull * u, min(8u, nc - 8u * u), unit_join(smv[j], ev[j]));
      }
    }
  }
  __syncthreads();
  const uint32_t m = s_m[0] + s_m[1] + s_m[2] + s_m[3];
  const uint64_t len_pad = b - a;
  uint32_t lo = 0, hi = 0, words = 0;
  uint64_t len = 0;
  if (m == 0u) {
    bad |= len_pad != 0u;
  } else if (len_pad < kRansHead) {
    bad = true;
  } else {
    lo = in[a];
    hi = in[a + 1];
    const uint16_t* hw = reinterpret_cast<const uint16_t*>(in + a);
    bad |= hi < lo || hw[1] != 0u;
    for (uint32_t h = 0; h < kParts; h++) {
      const uint32_t w = hw[2u + h];
      words += w;
      // a part codes its values exactly when it has a stream, which holds at least the states
      bad |= (s_m[h] == 0u) != (w == 0u) || (w != 0u && w < 2u * kRansStates);
      if (tid == 0) s_nw[h] = w;
    }
    len = kRansHead + 2u * uint64_t(hi >= lo ? hi - lo + 1u : 0u) + 2u * uint64_t(words);
    bad |= pad128(len) != len_pad;
  }
  if (part_sum_u32(bad ? 1u : 0u, s_w) != 0u) {
    if (tid == 0) err_slots[c] = uint32_t(CIERA_ERR_FORMAT);
    return;
  }
  const uint32_t span = hi - lo + 1u;
  bool pad_bad = false;
  if (m)
    for (uint64_t k = len + tid; k < len_pad; k += kPartThreads) pad_bad |= in[a + k] != 0u;
  // frequencies (one symbol per thread), then the slot table: thread t fills
  // slots 16 t .. 16 t + 15, the first symbol by binary search over the
  // cumulative counts, the rest by stepping
  uint32_t f = 0;
  if (m && tid >= lo && tid <= hi) {
    const uint64_t o = a + kRansHead + 2u * (tid - lo);
    f = uint32_t(in[o]) | (uint32_t(in[o + 1u]) << 8);
  }
  const uint32_t fsum = part_sum_u32(f, s_w);
  const uint32_t cum_incl = part_incl_scan_u32(f, s_w);
  s_f[tid] = f;
  s_cum[tid] = cum_incl - f;
  __syncthreads();
  const bool table_ok = (m == 0u) || fsum == kRansM;
  if (m && table_ok) {
    const uint32_t k0 = 16u * tid;
    uint32_t lo_s = 0, hi_s = 255u;
    while (lo_s < hi_s) {  // the first s with cum_s + f_s > k0
      const uint32_t mid = (lo_s + hi_s) >> 1;
      if (s_cum[mid] + s_f[mid] > k0) hi_s = mid; else lo_s = mid + 1u;
    }
    uint32_t s = lo_s, cs = s_cum[s], fs = s_f[s];
    for (uint32_t k = k0; k < k0 + 16u; k++) {
      while (cs + fs <= k) {  // ends: the counts sum to 4096 > k
        s++;
        cs = s_cum[s];
        fs = s_f[s];
      }
      s_dtab[k] = s | ((fs - 1u) << 8) | ((k - cs) << 20);
    }
  }
  __syncthreads();
  // Wave h decodes part h; each symbol goes straight to y (and, in ciera
  // mode, to the receiver cache) with its sign+mantissa byte, loaded
  // kRansWin steps ahead.
  bool okd = table_ok;
  if (mh && okd) {
    uint32_t so = kRansHead + 2u * span;  // the part's stream in the payload (bytes)
    for (uint32_t h = 0; h < wave; h++) so += 2u * s_nw[h];
    const uint32_t nw = s_nw[wave];
    // The part's words come through the wave's ring: payload block j (bytes
    // 1024 j .. 1024 j + 1023) sits in slot j mod 4.  Each group first stores
    // the block loaded during the group before, then loads the block two
    // past the one holding the next unread word (the last block at most).
    // A group reads at most 512 words (one block), so every word it reads is
    // in the ring: the unread word's block and the next were loaded earlier,
    // and the four slots hold them until then.  Lanes whose part of a block
    // lies past the payload read its last 16 bytes instead (never used).
    uint8_t* ring = s_ring[wave];
    const uint16_t* ring16 = reinterpret_cast<const uint16_t*>(ring);
    const uint32_t jmax = uint32_t((len_pad - 1u) / kRansBlock);
    const uint64_t gmax = a + len_pad - 16u;
    auto block_load = [&](uint32_t j) -> uint4 {
      const uint64_t ad = min(a + uint64_t(j) * kRansBlock + 16u * lane, gmax);
      return *reinterpret_cast<const uint4*>(in + ad);
    };
    auto block_store = [&](uint32_t j, uint4 v) {
      *reinterpret_cast<uint4*>(ring + (j & 3u) * kRansBlock + 16u * lane) = v;
    };
    auto word = [&](uint32_t k) -> uint32_t {  // word k of the part's stream
      const uint32_t o = so + 2u * k;
      return ring16[((o / kRansBlock) & 3u) * (kRansBlock / 2u) + (o % kRansBlock) / 2u];
    };
    {
      const uint32_t j0 = so / kRansBlock;
      const uint4 b0 = block_load(min(j0, jmax)), b1 = block_load(min(j0 + 1u, jmax)),
                  b2 = block_load(min(j0 + 2u, jmax));
      block_store(min(j0, jmax), b0);
      block_store(min(j0 + 1u, jmax), b1);
      block_store(min(j0 + 2u, jmax), b2);
      __builtin_amdgcn_wave_barrier();
    }
    const uint16_t* gl = s_gl[wave];
    uint8_t* sym = s_sym + wave * kRansWin * kRansStates;
    const uint32_t gmask = (1u << log2G) - 1u;
    constexpr uint32_t kGroup = kRansWin * kRansStates;
    auto value_of = [&](uint32_t i) -> uint32_t {  // chunk-relative value of the part's symbol i
      return kCiera ? ((uint32_t(gl[i >> log2G]) << log2G) | (i & gmask)) : (wave * kPartValues + i);
    };
    uint32_t xs = word(2u * lane) | (word(2u * lane + 1u) << 16);
    okd = xs >= kRansL;
    uint32_t q = 2u * kRansStates;
    auto want = [&]() -> uint32_t { return min((so + 2u * q) / kRansBlock + 2u, jmax); };
    uint32_t jp = want();
    uint4 pend = block_load(jp);
    auto decode = [&](uint32_t t, bool full) -> uint32_t {
      const bool act = full || t * kRansStates + lane < mh;
      uint32_t s = 0;
      if (act) {
        const uint32_t e = s_dtab[xs & (kRansM - 1u)];
        s = e & 0xFFu;
        xs = (((e >> 8) & 0xFFFu) + 1u) * (xs >> 12) + (e >> 20);
      }
      const bool need = act && xs < kRansL;
      const uint64_t mk = __ballot(need);
      // word q + (the lanes below that need one); a read past the part's
      // words stays inside the ring and fails the count check at the end
      const uint32_t kk = __builtin_amdgcn_mbcnt_hi(uint32_t(mk >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(mk), q));
      if (need) xs = (xs << 16) | word(kk);
      q = __builtin_amdgcn_readfirstlane(q + uint32_t(__popcll(mk)));  // uniform: keep it scalar
      return s;
    };
    // One group of kRansWin steps (512 symbols): the steps' symbols go to the
    // wave's LDS buffer; then lane l joins symbols 8 l .. 8 l + 7 of the
    // group (8 contiguous values through the granule list) with their
    // sign+mantissa bytes and writes them (and, in ciera mode, the receiver
    // cache) with one wide store.  The sign+mantissa bytes of a group are
    // loaded while the group before it decodes (two buffers take turns); the
    // last group, the only one that can be partial, goes on its own.
    auto group = [&](uint32_t g, uint2 smv, uint32_t vi, uint32_t cnt, bool full) {
      block_store(jp, pend);
      __builtin_amdgcn_wave_barrier();
      jp = want();
      pend = block_load(jp);
#pragma unroll
      for (uint32_t k = 0; k < kRansWin; k++) {
        const uint32_t t = g * kRansWin + k;
        if (full || t * kRansStates < mh) sym[k * kRansStates + lane] = uint8_t(decode(t, full));
      }
      __builtin_amdgcn_wave_barrier();
      const uint2 e = *reinterpret_cast<const uint2*>(sym + 8u * lane);
      __builtin_amdgcn_wave_barrier();
      store_unit(y, start + vi, cnt, unit_join(smv, e));
      if (kCiera) store_bytes8(cache + start + vi, cnt, e);
    };
    const uint32_t ng = cdiv(mh, kGroup);
    if (ng >= 2u) {
      // full groups: every lane has 8 values, so every load is issued
      auto fetch = [&](uint32_t g, uint2& smv, uint32_t& vi) {
        vi = value_of(g * kGroup + 8u * lane);
        smv = *reinterpret_cast<const uint2*>(in + sm_pos + start + vi);
      };
      uint2 sa, sb;
      uint32_t va, vb;
      uint32_t g = 0;
      fetch(0u, sa, va);
      while (true) {
        fetch(min(g + 1u, ng - 2u), sb, vb);
        group(g, sa, va, 8u, true);
        if (++g == ng - 1u) break;
        fetch(min(g + 1u, ng - 2u), sa, va);
        group(g, sb, vb, 8u, true);
        if (++g == ng - 1u) break;
      }
    }
    {
      const uint32_t i0 = (ng - 1u) * kGroup + 8u * lane;
      const uint32_t cnt = (i0 < mh) ? min(8u, mh - i0) : 0u;
      const uint32_t vi = value_of(cnt ? i0 : 0u);
      const uint2 smv = cnt ? load_bytes8(in + sm_pos + start + vi, cnt) : make_uint2(0u, 0u);
      group(ng - 1u, smv, vi, cnt, false);
    }
    okd = okd && q == nw && xs == kRansL;
  }
  const bool dec_ok = part_sum_u32((okd && !pad_bad) ? 0u : 1u, s_w) == 0u;
  if (tid == 0) err_slots[c] = dec_ok ? 0u : uint32_t(CIERA_ERR_FORMAT);
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
  return table_end(nchunks) + full * chunk_max_bytes(kChunk, B) + (rem ? chunk_max_bytes(rem, B) : 0u);
}

// k_plan's shape: at least kPlanMinChunks chunks per group unless that takes
// more than kPlanMaxGroups (or max_groups, if nonzero) groups; no group is
// empty.
void plan_shape(uint64_t nchunks, uint32_t max_groups, uint64_t& per, uint32_t& groups) {
  const uint32_t cap = (max_groups && max_groups < kPlanMaxGroups) ? max_groups : kPlanMaxGroups;
  uint64_t g = cdiv(nchunks, kPlanMinChunks);
  if (g < 1u) g = 1u;
  if (g > cap) g = cap;
  per = nchunks ? cdiv(nchunks, g) : 1u;
  groups = nchunks ? uint32_t(cdiv(nchunks, per)) : 1u;
}

ciera_status launch_status() {
  return hipGetLastError() == hipSuccess ? CIERA_OK : CIERA_ERR_HIP;
}

// Kernel timing on request: each launch takes the next (start, stop) pair of
// the calling thread's queue, if any, and has the runtime record the pair at
// the kernel's own start and end.
thread_local std::vector<hipEvent_t> t_events;
thread_local size_t t_next_event = 0;

template <typename... P, typename... A>
void launch(void (*kernel)(P...), dim3 grid, dim3 block, hipStream_t stream, A... args) {
  if (t_next_event + 2u <= t_events.size()) {
    hipEvent_t start = t_events[t_next_event], stop = t_events[t_next_event + 1u];
    t_next_event += 2u;
    hipExtLaunchKernelGGL(kernel, grid, block, 0u, stream, start, stop, 0u, static_cast<P>(args)...);
  } else {
    hipLaunchKernelGGL(kernel, grid, block, 0, stream, static_cast<P>(args)...);
  }
}

// d_hash non-null: ciera mode with the block-hash sender state instead of the
// exponent cache (d_cache unused).
// d_e0: a window base in device memory (the single-read entry points on
// tensors of at most kSelfPlanChunks chunks), else null.
ciera_status encode_impl(const void* d_x, uint64_t n, uint32_t B, uint8_t* d_cache, void* d_out,
                         uint64_t out_capacity, void* d_ws, uint64_t ws_bytes, uint64_t* d_out_size,
                         int e0_override, uint32_t plan_groups, hipStream_t stream, void* d_hash = nullptr,
                         const uint8_t* d_e0 = nullptr) {
  const bool ciera = B != 0u;
  const bool hashed = d_hash != nullptr;
  if (n > kMaxN) return CIERA_ERR_ARG;
  if (ciera && !valid_block(B)) return CIERA_ERR_ARG;
  if (e0_override < -1 || e0_override > int(kMaxE0)) return CIERA_ERR_ARG;
  if (!d_out || !d_ws || !d_out_size || !aligned16(d_out) || !aligned16(d_ws)) return CIERA_ERR_ARG;
  if ((reinterpret_cast<uintptr_t>(d_out_size) & 7u) != 0u) return CIERA_ERR_ARG;
  if (n > 0 && (!d_x || !aligned16(d_x))) return CIERA_ERR_ARG;
  if (ciera && !hashed && n > 0 && (!d_cache || !aligned16(d_cache))) return CIERA_ERR_ARG;
  if (hashed && (!ciera || !aligned16(d_hash))) return CIERA_ERR_ARG;
  if (out_capacity < max_size(n, B)) return CIERA_ERR_CAPACITY;
  const uint64_t nchunks = cdiv(n, kChunk);
  if (ws_bytes < ws_layout(nchunks).total) return CIERA_ERR_WORKSPACE;
  // A tensor of at most kSelfPlanChunks chunks (one planning group) is
  // planned by the write kernel itself, unless a planner shape is forced.
  // Its k_stats then runs one workgroup per slice of a part (kSlices per
  // part, one record each), except for blocks that span slices.
  const bool self_plan = plan_groups == 0u && nchunks >= 1u && nchunks <= kSelfPlanChunks && !(hashed && B > kPartValues);
  const bool stats_sliced = self_plan && (!ciera || B <= 8u * (kPartUnits / kSlices));
  static_assert(kSelfPlanChunks <= kSliceChunks, "the workspace has a record per slice");
  if (d_e0 && (!self_plan || hashed || e0_override >= 0)) return CIERA_ERR_ARG;
  Ws ws = ws_bind(d_ws, nchunks);
  ws.ss = stats_sliced ? kSlices : 1u;
  ws.e0_src = d_e0;
  const uint32_t lb = ciera ? log2u(B) : 0u;
  uint64_t* hcache = static_cast<uint64_t*>(d_hash);
  const uint16_t* x = static_cast<const uint16_t*>(d_x);
  uint8_t* out = static_cast<uint8_t*>(d_out);
  (void)hipGetLastError();
  if (nchunks) {
    const dim3 grid(uint32_t(nchunks * kParts)), sgrid(uint32_t(nchunks * kParts * kSlices));
    if (hashed && stats_sliced)
      launch(k_stats<true, true, kSlices>, sgrid, dim3(kPartThreads), stream, x, n, static_cast<uint8_t*>(d_hash), lb,
             ws);
    else if (hashed)
      launch(k_stats<true, true, 1u>, grid, dim3(kPartThreads), stream, x, n, static_cast<uint8_t*>(d_hash), lb, ws);
    else if (ciera && stats_sliced)
      launch(k_stats<true, false, kSlices>, sgrid, dim3(kPartThreads), stream, x, n, d_cache, lb, ws);
    else if (ciera)
      launch(k_stats<true, false, 1u>, grid, dim3(kPartThreads), stream, x, n, d_cache, lb, ws);
    else if (stats_sliced)
      launch(k_stats<false, false, kSlices>, sgrid, dim3(kPartThreads), stream, x, n, nullptr, 0u, ws);
    else
      launch(k_stats<false, false, 1u>, grid, dim3(kPartThreads), stream, x, n, nullptr, 0u, ws);
  }
  if (!self_plan) {
    uint64_t per = 0;
    uint32_t groups = 0;
    plan_shape(nchunks, plan_groups, per, groups);
    launch(k_sums, dim3(groups), dim3(kPlanThreads), stream, nchunks, per, ws);
    if (hashed && B > kPartValues)
      launch(k_plan<true>, dim3(groups), dim3(kPlanThreads), stream, n, nchunks, per, B, e0_override, out, d_out_size,
             hcache, ws);
    else
      launch(k_plan<false>, dim3(groups), dim3(kPlanThreads), stream, n, nchunks, per, B, e0_override, out,
             d_out_size, nullptr, ws);
  }
  if (nchunks) {
    // a self-planned tensor is small: kSlices workgroups per part
    const dim3 grid(uint32_t(nchunks * kParts));
    const dim3 sgrid(uint32_t(nchunks * kParts * kSlices));
    if (ciera && self_plan)
      launch(k_write<true, true, kSlices>, sgrid, dim3(kPartThreads), stream, x, n, lb, out, out_capacity, d_out_size,
             e0_override, ws);
    else if (ciera)
      launch(k_write<true, false, 1u>, grid, dim3(kPartThreads), stream, x, n, lb, out, out_capacity, d_out_size,
             e0_override, ws);
    else if (self_plan)
      launch(k_write<false, true, kSlices>, sgrid, dim3(kPartThreads), stream, x, n, 0u, out, out_capacity,
             d_out_size, e0_override, ws);
    else
      launch(k_write<false, false, 1u>, grid, dim3(kPartThreads), stream, x, n, 0u, out, out_capacity, d_out_size,
             e0_override, ws);
  }
  return launch_status();
}

ciera_status encode_known_e0_impl(const void* d_x, uint64_t n, uint32_t B, uint8_t* d_cache, const uint8_t* d_e0,
                                  void* d_out, uint64_t out_capacity, void* d_ws, uint64_t ws_bytes,
                                  uint64_t* d_out_size, hipStream_t stream) {
  const bool ciera = B != 0u;
  if (n > kMaxSingleReadN) return CIERA_ERR_ARG;
  if (ciera && !valid_block(B)) return CIERA_ERR_ARG;
  if (!d_e0 || !d_out || !d_ws || !d_out_size || !aligned16(d_out) || !aligned16(d_ws)) return CIERA_ERR_ARG;
  if ((reinterpret_cast<uintptr_t>(d_out_size) & 7u) != 0u) return CIERA_ERR_ARG;
  if (n > 0 && (!d_x || !aligned16(d_x))) return CIERA_ERR_ARG;
  if (ciera && n > 0 && (!d_cache || !aligned16(d_cache))) return CIERA_ERR_ARG;
  if (out_capacity < max_size(n, B)) return CIERA_ERR_CAPACITY;
  const uint64_t nchunks = cdiv(n, kChunk);
  if (ws_bytes < ws_layout(nchunks).total) return CIERA_ERR_WORKSPACE;
  // A tensor of at most kSelfPlanChunks chunks (2 MiB of input, which the
  // MALL holds) runs the self-planned two-launch encode with the given
  // window base: faster there than one read with waits between workgroups.
  if (nchunks >= 1u && nchunks <= kSelfPlanChunks)
    return encode_impl(d_x, n, B, d_cache, d_out, out_capacity, d_ws, ws_bytes, d_out_size, -1, 0u, stream, nullptr,
                       d_e0);
  const Ws ws = ws_bind(d_ws, nchunks);
  const uint16_t* x = static_cast<const uint16_t*>(d_x);
  uint8_t* out = static_cast<uint8_t*>(d_out);
  (void)hipGetLastError();
  const uint64_t prep_groups = cdiv(nchunks * kParts, kThreads);
  launch(k_prep1, dim3(uint32_t(prep_groups < 1u ? 1u : (prep_groups > 1024u ? 1024u : prep_groups))), dim3(kThreads),
         stream, n, nchunks, B, d_e0, out, d_out_size, ws);
  if (nchunks) {
    if (ciera)
      launch(k_write1<true>, dim3(uint32_t(nchunks * kParts)), dim3(kPartThreads), stream, x, n, nchunks, log2u(B),
             d_cache, out, d_out_size, ws);
    else
      launch(k_write1<false>, dim3(uint32_t(nchunks * kParts)), dim3(kPartThreads), stream, x, n, nchunks, 0u,
             nullptr, out, d_out_size, ws);
  }
  return launch_status();
}

// rANS modes: the workspace of the 3-bit path followed by, per chunk, the
// look-back word, the coded-count record and a payload scratch slot.
uint64_t rans_ws_size(uint64_t n) {
  const uint64_t nchunks = cdiv(n, kChunk);
  return ws_layout(nchunks).total + align256(8u * kRstatStride * nchunks) + align256(8u * nchunks) +
         nchunks * uint64_t(kRansSlot);
}

Ws rans_ws_bind(void* base, uint64_t n) {
  const uint64_t nchunks = cdiv(n, kChunk);
  Ws w = ws_bind(base, nchunks);
  uint8_t* b = static_cast<uint8_t*>(base) + ws_layout(nchunks).total;
  w.rstat = reinterpret_cast<uint64_t*>(b);
  w.rinfo = reinterpret_cast<uint64_t*>(b + align256(8u * kRstatStride * nchunks));
  w.rslot = b + align256(8u * kRstatStride * nchunks) + align256(8u * nchunks);
  return w;
}

uint64_t rans_max_size(uint64_t n, uint32_t B) {
  const uint64_t nchunks = cdiv(n, kChunk);
  uint64_t size = rans_pay_pos(n, nchunks, B != 0u);
  const uint64_t full = n / kChunk, rem = n % kChunk;
  size += full * pad128(rans_chunk_max(kChunk));
  if (rem) size += pad128(rans_chunk_max(rem));
  return size;
}

ciera_status encode_rans_impl(const void* d_x, uint64_t n, uint32_t B, uint8_t* d_cache, void* d_out,
                              uint64_t out_capacity, void* d_ws, uint64_t ws_bytes, uint64_t* d_out_size,
                              hipStream_t stream) {
  const bool ciera = B != 0u;
  if (n > kMaxN) return CIERA_ERR_ARG;
  if (ciera && !valid_block(B)) return CIERA_ERR_ARG;
  if (!d_out || !d_ws || !d_out_size || !aligned16(d_out) || !aligned16(d_ws)) return CIERA_ERR_ARG;
  if ((reinterpret_cast<uintptr_t>(d_out_size) & 7u) != 0u) return CIERA_ERR_ARG;
  if (n > 0 && (!d_x || !aligned16(d_x))) return CIERA_ERR_ARG;
  if (ciera && n > 0 && (!d_cache || !aligned16(d_cache))) return CIERA_ERR_ARG;
  if (out_capacity < rans_max_size(n, B)) return CIERA_ERR_CAPACITY;
  if (ws_bytes < rans_ws_size(n)) return CIERA_ERR_WORKSPACE;
  const uint64_t nchunks = cdiv(n, kChunk);
  const Ws ws = rans_ws_bind(d_ws, n);
  const uint32_t lb = ciera ? log2u(B) : 0u;
  const uint16_t* x = static_cast<const uint16_t*>(d_x);
  uint8_t* out = static_cast<uint8_t*>(d_out);
  const uint32_t parts = uint32_t(nchunks * kParts);
  (void)hipGetLastError();
  if (nchunks) {
    if (ciera) {
      launch(k_stats<true, false, 1u>, dim3(parts), dim3(kPartThreads), stream, x, n, d_cache, lb, ws);
      launch(k_rans_enc<true>, dim3(uint32_t(nchunks)), dim3(kPartThreads), stream, x, n, nchunks, lb, out, ws);
    } else {
      launch(k_stats<false, false, 1u>, dim3(parts), dim3(kPartThreads), stream, x, n, nullptr, 0u, ws);
      launch(k_rans_enc<false>, dim3(uint32_t(nchunks)), dim3(kPartThreads), stream, x, n, nchunks, 0u, out, ws);
    }
  }
  launch(k_rans_finish, dim3(1), dim3(kThreads), stream, n, nchunks, B, out, d_out_size, ws);
  return launch_status();
}

ciera_status decode_rans_impl(const void* d_in, uint64_t in_size, void* d_y, uint64_t n, uint32_t B,
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
    launch(k_rans_dec<true>, dim3(grid), dim3(kPartThreads), stream, in, in_size, y, n, nchunks, log2u(B), d_cache,
           &ws.ctrl->n_err_slots, ws.err);
  else
    launch(k_rans_dec<false>, dim3(grid), dim3(kPartThreads), stream, in, in_size, y, n, nchunks, 0u, nullptr,
           &ws.ctrl->n_err_slots, ws.err);
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
  const bool sliced = nchunks <= kSliceChunks;
  const uint32_t grid = uint32_t(nchunks ? nchunks * kParts * (sliced ? kSlices : 1u) : 1u);
  const uint8_t* in = static_cast<const uint8_t*>(d_in);
  uint16_t* y = static_cast<uint16_t*>(d_y);
  const uint32_t lb = ciera ? log2u(B) : 0u;
  uint8_t* cache = ciera ? d_cache : nullptr;
  (void)hipGetLastError();
  if (ciera && sliced)
    launch(k_decode<true, kSlices>, dim3(grid), dim3(kPartThreads), stream, in, in_size, y, n, nchunks, lb, cache,
           &ws.ctrl->n_err_slots, ws.err);
  else if (ciera)
    launch(k_decode<true, 1u>, dim3(grid), dim3(kPartThreads), stream, in, in_size, y, n, nchunks, lb, cache,
           &ws.ctrl->n_err_slots, ws.err);
  else if (sliced)
    launch(k_decode<false, kSlices>, dim3(grid), dim3(kPartThreads), stream, in, in_size, y, n, nchunks, lb, cache,
           &ws.ctrl->n_err_slots, ws.err);
  else
    launch(k_decode<false, 1u>, dim3(grid), dim3(kPartThreads), stream, in, in_size, y, n, nchunks, lb, cache,
           &ws.ctrl->n_err_slots, ws.err);
  return launch_status();
}

// Speculative encode: the single-read write with a hinted window base that
// also keeps k_stats' records, then k_sums and k_check (the window the
// variance gives, against the hint), then the two-pass encode's k_stats (with
// the recorded change bits), k_plan and k_write, which return at once when
// the hint was right.  Either way the stream, the cache and *d_out_size are
// those of the regular encode.  Tensors of at most kSelfPlanChunks chunks, or
// above the single-read limit, take the regular encode.
ciera_status encode_spec_impl(const void* d_x, uint64_t n, uint32_t B, uint8_t* d_cache, const uint8_t* d_hint,
                              void* d_out, uint64_t out_capacity, void* d_ws, uint64_t ws_bytes, uint64_t* d_out_size,
                              hipStream_t stream) {
  const bool ciera = B != 0u;
  if (!d_hint) return CIERA_ERR_ARG;
  const uint64_t nchunks = cdiv(n, kChunk);
  if (nchunks <= kSelfPlanChunks || n > kMaxSingleReadN)
    return encode_impl(d_x, n, B, d_cache, d_out, out_capacity, d_ws, ws_bytes, d_out_size, -1, 0u, stream);
  if (ciera && !valid_block(B)) return CIERA_ERR_ARG;
  if (!d_out || !d_ws || !d_out_size || !aligned16(d_out) || !aligned16(d_ws)) return CIERA_ERR_ARG;
  if ((reinterpret_cast<uintptr_t>(d_out_size) & 7u) != 0u) return CIERA_ERR_ARG;
  if (!d_x || !aligned16(d_x)) return CIERA_ERR_ARG;
  if (ciera && (!d_cache || !aligned16(d_cache))) return CIERA_ERR_ARG;
  if (out_capacity < max_size(n, B)) return CIERA_ERR_CAPACITY;
  if (ws_bytes < ws_layout(nchunks).total) return CIERA_ERR_WORKSPACE;
  const Ws ws = ws_bind(d_ws, nchunks);
  Ws wsf = ws;
  wsf.spec = 1u;  // the fallback launches
  const uint16_t* x = static_cast<const uint16_t*>(d_x);
  uint8_t* out = static_cast<uint8_t*>(d_out);
  const uint32_t lb = ciera ? log2u(B) : 0u;
  const dim3 grid(uint32_t(nchunks * kParts));
  uint64_t per = 0;
  uint32_t groups = 0;
  plan_shape(nchunks, 0u, per, groups);
  (void)hipGetLastError();
  const uint64_t prep_groups = cdiv(nchunks * kParts, kThreads);
  launch(k_prep1, dim3(uint32_t(prep_groups > 1024u ? 1024u : prep_groups)), dim3(kThreads), stream, n, nchunks, B,
         d_hint, out, d_out_size, ws);
  if (ciera)
    launch(k_write1<true, true>, grid, dim3(kPartThreads), stream, x, n, nchunks, lb, d_cache, out, d_out_size, ws);
  else
    launch(k_write1<false, true>, grid, dim3(kPartThreads), stream, x, n, nchunks, 0u, nullptr, out, d_out_size, ws);
  launch(k_sums, dim3(groups), dim3(kPlanThreads), stream, nchunks, per, ws);
  launch(k_check, dim3(1), dim3(kPlanThreads), stream, groups, ws);
  if (ciera) {
    launch(k_stats<true, false, 1u, true>, grid, dim3(kPartThreads), stream, x, n, d_cache, lb, wsf);
    launch(k_plan<false>, dim3(groups), dim3(kPlanThreads), stream, n, nchunks, per, B, -1, out, d_out_size, nullptr,
           wsf);
    launch(k_write<true, false, 1u>, grid, dim3(kPartThreads), stream, x, n, lb, out, out_capacity, d_out_size, -1,
           wsf);
  } else {
    launch(k_stats<false, false, 1u, true>, grid, dim3(kPartThreads), stream, x, n, nullptr, 0u, wsf);
    launch(k_plan<false>, dim3(groups), dim3(kPlanThreads), stream, n, nchunks, per, 0u, -1, out, d_out_size, nullptr,
           wsf);
    launch(k_write<false, false, 1u>, grid, dim3(kPartThreads), stream, x, n, 0u, out, out_capacity, d_out_size, -1,
           wsf);
  }
  return launch_status();
}

// Batch decode: k streams of one n and B in one launch of k_decode_batch,
// each stream with the single decode's workgroups, their status words one
// after the other after the control block.
uint64_t decode_workgroups(uint64_t nchunks) {
  return nchunks ? nchunks * kParts * (nchunks <= kSliceChunks ? kSlices : 1u) : 1u;
}
uint64_t decode_batch_ws_bytes(uint64_t nchunks, uint32_t k) {
  return align256(sizeof(Ctrl) + 4u * uint64_t(k) * decode_workgroups(nchunks));
}

ciera_status decode_batch_impl(uint32_t k, const void* const* d_in, const uint64_t* in_size, void* const* d_y,
                               uint64_t n, uint32_t B, uint8_t* const* d_cache, void* d_ws, uint64_t ws_bytes,
                               hipStream_t stream) {
  const bool ciera = B != 0u;
  if (k == 0u || k > kDecodeBatchMax || !d_in || !in_size || !d_y) return CIERA_ERR_ARG;
  if (n > kMaxN / k) return CIERA_ERR_ARG;
  if (ciera && (!valid_block(B) || !d_cache)) return CIERA_ERR_ARG;
  if (!d_ws || !aligned16(d_ws)) return CIERA_ERR_ARG;
  DecodeStreams st;
  memset(&st, 0, sizeof(st));
  for (uint32_t i = 0; i < k; i++) {
    if (!d_in[i] || !aligned16(d_in[i])) return CIERA_ERR_ARG;
    if (n > 0 && (!d_y[i] || !aligned16(d_y[i]))) return CIERA_ERR_ARG;
    if (ciera && n > 0 && (!d_cache[i] || !aligned16(d_cache[i]))) return CIERA_ERR_ARG;
    st.in[i] = static_cast<const uint8_t*>(d_in[i]);
    st.in_size[i] = in_size[i];
    st.y[i] = static_cast<uint16_t*>(d_y[i]);
    st.cache[i] = ciera ? d_cache[i] : nullptr;
  }
  const uint64_t nchunks = cdiv(n, kChunk);
  if (ws_bytes < decode_batch_ws_bytes(nchunks, k)) return CIERA_ERR_WORKSPACE;
  uint64_t* n_err_slots = &static_cast<Ctrl*>(d_ws)->n_err_slots;
  uint32_t* err = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(d_ws) + sizeof(Ctrl));
  const uint32_t per = uint32_t(decode_workgroups(nchunks));
  const dim3 grid(k * per);
  const bool sliced = nchunks <= kSliceChunks;
  const uint32_t lb = ciera ? log2u(B) : 0u;
  (void)hipGetLastError();
  if (ciera && sliced)
    launch(k_decode_batch<true, kSlices>, grid, dim3(kPartThreads), stream, st, per, n, nchunks, lb, n_err_slots, err);
  else if (ciera)
    launch(k_decode_batch<true, 1u>, grid, dim3(kPartThreads), stream, st, per, n, nchunks, lb, n_err_slots, err);
  else if (sliced)
    launch(k_decode_batch<false, kSlices>, grid, dim3(kPartThreads), stream, st, per, n, nchunks, lb, n_err_slots,
           err);
  else
    launch(k_decode_batch<false, 1u>, grid, dim3(kPartThreads), stream, st, per, n, nchunks, lb, n_err_slots, err);
  return launch_status();
}

// ------------------------------------------------------------------ no-allocation entry point
// ciera_encode_noalloc runs ciera_encode's kernels on a workspace that lives
// in this array instead of a caller's buffer.  Each GPU holds its own copy;
// host code must use the address hipGetSymbolAddress returns for the current
// device, never the array's name (a host-side stand-in).
constexpr uint64_t kScratchBytes = 6ull << 20;
constexpr uint64_t kNoAllocMaxN = CIERA_NOALLOC_MAX_N;  // 2048 chunks: ws_layout needs about 5.5 MB
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

}  // namespace

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

// The scratch array's device address on the current device, looked up once
// per device (with that device current) and kept.
ciera_status scratch_on_current_device(void** ptr_out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return CIERA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return CIERA_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *ptr_out = g_scratch_ptr[dev];
  return CIERA_OK;
}

}  // namespace

extern "C" {

ciera_status ciera_encode_noalloc(const void* d_x, uint64_t n, uint32_t B, uint8_t* d_prev_exp, void* d_out,
                                  uint64_t out_capacity, uint64_t* d_out_size, hipStream_t stream) {
  if (B == 0u || !valid_block(B)) return CIERA_ERR_ARG;
  if (n > kNoAllocMaxN || ws_layout(cdiv(n, kChunk)).total > kScratchBytes) return CIERA_ERR_WORKSPACE;
  void* ws = nullptr;
  const ciera_status st = scratch_on_current_device(&ws);
  if (st != CIERA_OK) return st;
  return encode_impl(d_x, n, B, d_prev_exp, d_out, out_capacity, ws, kScratchBytes, d_out_size, -1, 0u, stream);
}

ciera_status zip3_encode_spec(const void* d_x, uint64_t n, const uint8_t* d_hint, void* d_out, uint64_t out_capacity,
                              void* d_ws, uint64_t ws_bytes, uint64_t* d_out_size, hipStream_t stream) {
  if (n > kMaxN) return CIERA_ERR_ARG;
  return encode_spec_impl(d_x, n, 0u, nullptr, d_hint, d_out, out_capacity, d_ws, ws_bytes, d_out_size, stream);
}

ciera_status ciera_encode_spec(const void* d_x, uint64_t n, uint32_t B, uint8_t* d_prev_exp, const uint8_t* d_hint,
                               void* d_out, uint64_t out_capacity, void* d_ws, uint64_t ws_bytes, uint64_t* d_out_size,
                               hipStream_t stream) {
  if (B == 0u || n > kMaxN) return CIERA_ERR_ARG;
  return encode_spec_impl(d_x, n, B, d_prev_exp, d_hint, d_out, out_capacity, d_ws, ws_bytes, d_out_size, stream);
}

uint64_t decode_batch_workspace_size(uint64_t n, uint32_t k) {
  return (k == 0u || k > kDecodeBatchMax || n > kMaxN / k) ? 0u : decode_batch_ws_bytes(cdiv(n, kChunk), k);
}

ciera_status zip3_decode_batch(uint32_t k, const void* const* d_in, const uint64_t* in_size, void* const* d_y,
                               uint64_t n, void* d_ws, uint64_t ws_bytes, hipStream_t stream) {
  return decode_batch_impl(k, d_in, in_size, d_y, n, 0u, nullptr, d_ws, ws_bytes, stream);
}

ciera_status ciera_decode_batch(uint32_t k, const void* const* d_in, const uint64_t* in_size, void* const* d_y,
                                uint64_t n, uint32_t B, uint8_t* const* d_prev_exp, void* d_ws, uint64_t ws_bytes,
                                hipStream_t stream) {
  if (B == 0u) return CIERA_ERR_ARG;
  return decode_batch_impl(k, d_in, in_size, d_y, n, B, d_prev_exp, d_ws, ws_bytes, stream);
}

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
  return encode_impl(d_x, n, 0u, nullptr, d_out, out_capacity, d_ws, ws_bytes, d_out_size, -1, 0u, stream);
}

ciera_status zip3_encode_ex(const void* d_x, uint64_t n, void* d_out, uint64_t out_capacity, void* d_ws,
                            uint64_t ws_bytes, uint64_t* d_out_size, int e0_override, uint32_t plan_groups,
                            hipStream_t stream) {
  return encode_impl(d_x, n, 0u, nullptr, d_out, out_capacity, d_ws, ws_bytes, d_out_size, e0_override,
                     plan_groups, stream);
}

ciera_status zip3_decode(const void* d_in, uint64_t in_size, void* d_y, uint64_t n, void* d_ws,
                         uint64_t ws_bytes, hipStream_t stream) {
  return decode_impl(d_in, in_size, d_y, n, 0u, nullptr, d_ws, ws_bytes, stream);
}

ciera_status ciera_encode(const void* d_x, uint64_t n, uint32_t B, uint8_t* d_prev_exp, void* d_out,
                          uint64_t out_capacity, void* d_ws, uint64_t ws_bytes, uint64_t* d_out_size,
                          hipStream_t stream) {
  if (B == 0u) return CIERA_ERR_ARG;
  return encode_impl(d_x, n, B, d_prev_exp, d_out, out_capacity, d_ws, ws_bytes, d_out_size, -1, 0u, stream);
}

ciera_status ciera_encode_ex(const void* d_x, uint64_t n, uint32_t B, uint8_t* d_prev_exp, void* d_out,
                             uint64_t out_capacity, void* d_ws, uint64_t ws_bytes, uint64_t* d_out_size,
                             int e0_override, uint32_t plan_groups, hipStream_t stream) {
  if (B == 0u) return CIERA_ERR_ARG;
  return encode_impl(d_x, n, B, d_prev_exp, d_out, out_capacity, d_ws, ws_bytes, d_out_size, e0_override,
                     plan_groups, stream);
}

uint64_t rans_max_encoded_size(uint64_t n, uint32_t B) {
  return (n > kMaxN || (B && !valid_block(B))) ? 0u : rans_max_size(n, B);
}

uint64_t rans_workspace_size(uint64_t n, uint32_t B) {
  return (n > kMaxN || (B && !valid_block(B))) ? 0u : rans_ws_size(n);
}

ciera_status zip3_encode_rans(const void* d_x, uint64_t n, void* d_out, uint64_t out_capacity, void* d_ws,
                              uint64_t ws_bytes, uint64_t* d_out_size, hipStream_t stream) {
  return encode_rans_impl(d_x, n, 0u, nullptr, d_out, out_capacity, d_ws, ws_bytes, d_out_size, stream);
}

ciera_status zip3_decode_rans(const void* d_in, uint64_t in_size, void* d_y, uint64_t n, void* d_ws,
                              uint64_t ws_bytes, hipStream_t stream) {
  return decode_rans_impl(d_in, in_size, d_y, n, 0u, nullptr, d_ws, ws_bytes, stream);
}

ciera_status ciera_encode_rans(const void* d_x, uint64_t n, uint32_t B, uint8_t* d_prev_exp, void* d_out,
                               uint64_t out_capacity, void* d_ws, uint64_t ws_bytes, uint64_t* d_out_size,
                               hipStream_t stream) {
  if (B == 0u) return CIERA_ERR_ARG;
  return encode_rans_impl(d_x, n, B, d_prev_exp, d_out, out_capacity, d_ws, ws_bytes, d_out_size, stream);
}

ciera_status ciera_decode_rans(const void* d_in, uint64_t in_size, void* d_y, uint64_t n, uint32_t B,
                               uint8_t* d_prev_exp, void* d_ws, uint64_t ws_bytes, hipStream_t stream) {
  if (B == 0u) return CIERA_ERR_ARG;
  return decode_rans_impl(d_in, in_size, d_y, n, B, d_prev_exp, d_ws, ws_bytes, stream);
}

uint64_t ciera_hash_cache_size(uint64_t n, uint32_t B) {
  return (n > kMaxN || !valid_block(B)) ? 0u : 16u * cdiv(n, B);
}

ciera_status ciera_encode_hashed(const void* d_x, uint64_t n, uint32_t B, void* d_hash_cache, void* d_out,
                                 uint64_t out_capacity, void* d_ws, uint64_t ws_bytes, uint64_t* d_out_size,
                                 hipStream_t stream) {
  if (B == 0u || (!d_hash_cache && n > 0)) return CIERA_ERR_ARG;
  return encode_impl(d_x, n, B, nullptr, d_out, out_capacity, d_ws, ws_bytes, d_out_size, -1, 0u, stream,
                     d_hash_cache);
}

ciera_status ciera_decode(const void* d_in, uint64_t in_size, void* d_y, uint64_t n, uint32_t B,
                          uint8_t* d_prev_exp, void* d_ws, uint64_t ws_bytes, hipStream_t stream) {
  if (B == 0u) return CIERA_ERR_ARG;
  return decode_impl(d_in, in_size, d_y, n, B, d_prev_exp, d_ws, ws_bytes, stream);
}

ciera_status zip3_encode_e0(const void* d_x, uint64_t n, const uint8_t* d_e0, void* d_out, uint64_t out_capacity,
                           void* d_ws, uint64_t ws_bytes, uint64_t* d_out_size, hipStream_t stream) {
  return encode_known_e0_impl(d_x, n, 0u, nullptr, d_e0, d_out, out_capacity, d_ws, ws_bytes, d_out_size, stream);
}

ciera_status ciera_encode_e0(const void* d_x, uint64_t n, uint32_t B, uint8_t* d_prev_exp, const uint8_t* d_e0,
                             void* d_out, uint64_t out_capacity, void* d_ws, uint64_t ws_bytes, uint64_t* d_out_size,
                             hipStream_t stream) {
  if (B == 0u) return CIERA_ERR_ARG;
  return encode_known_e0_impl(d_x, n, B, d_prev_exp, d_e0, d_out, out_capacity, d_ws, ws_bytes, d_out_size, stream);
}

ciera_status ciera_read_error(const void* d_ws, hipStream_t stream) {
  if (!d_ws) return CIERA_ERR_ARG;
  const Ctrl* ctrl = static_cast<const Ctrl*>(d_ws);
  uint64_t slots = 0;
  if (hipMemcpyAsync(&slots, &ctrl->n_err_slots, sizeof(slots), hipMemcpyDeviceToHost, stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess)
    return CIERA_ERR_HIP;
  if (slots == 0u) return CIERA_OK;
  if (slots > kParts * cdiv(kMaxN, kChunk)) return CIERA_ERR_INTERNAL;
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

uint32_t ciera_set_wait_limit(uint32_t polls) {
  return g_wait_limit.exchange(polls ? polls : kSpinLimit, std::memory_order_relaxed);
}

ciera_status ciera_time_kernels(void* const* events, uint32_t n_pairs) {
  if (n_pairs && !events) return CIERA_ERR_ARG;
  for (uint32_t i = 0; i < 2u * n_pairs; i++)
    if (!events[i]) return CIERA_ERR_ARG;
  const hipEvent_t* ev = reinterpret_cast<const hipEvent_t*>(events);
  t_events.assign(ev, ev + 2u * n_pairs);
  t_next_event = 0;
  return CIERA_OK;
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
