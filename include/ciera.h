/*
 * ciera.h -- C ABI of the lossless BF16 codec for MI355X (gfx950).
 *
 * The codec turns a BF16 tensor into a byte stream and back, bit for bit:
 *
 *  - every value is split into a sign+mantissa byte and its 8-bit exponent
 *    (ZipCCL research digest, section 3.1; CIERA page, section 3.1);
 *  - exponents are coded in 3 bits against a 7-binade window whose base E0 is
 *    chosen from the tensor's standard deviation, with code 0 plus the raw
 *    exponent (an "escape") for values outside it (ZipCCL digest, section
 *    3.1, the P_win and x_opt equations and Figure 2);
 *  - in ciera mode, blocks of B values whose exponents all equal the previous
 *    iteration's are flagged unchanged in a bitmap and send no exponents; the
 *    receiver takes them from its own cache (CIERA page, sections 3.1-3.2);
 *  - the stream is cut into chunks of 65,536 input values, each written as a
 *    self-contained segment whose sections (sign+mantissa, bitmap, three code
 *    bit-planes, escapes) start on 128-byte boundaries (ZipCCL digest,
 *    section 3.1 last paragraph and Figure 1).
 *
 * Stream layout (little-endian; all padding and unnamed bytes are zero):
 *   header (128 B): "ZIP3"|"CIER", u16 version=1, u8 mode (0 zip3, 1 ciera),
 *     u8 E0, u64 n, u32 B (0 in zip3), u32 C=65536, u64 nchunks,
 *     u64 total_bytes, u64 n_changed_blocks, u64 n_escapes;
 *   chunk table at byte 128: nchunks+1 u64 absolute offsets;
 *   escape index right after it: per chunk four u16, the number of escapes
 *     among the chunk's values before value 0, 16384, 32768 and 49152 of
 *     the chunk (a seek index: each quarter decodes on its own); table and
 *     index padded together to 128;
 *   per chunk: sm[n_c] | bitmap[ceil(nb_c/8)] (ciera) | plane0..2[P_c] |
 *     escapes[n_esc_c], each padded to 128.  Plane b holds bit b of the code
 *     of slot t in bit (t&7) of byte (t>>3).  zip3: slot t = value t of the
 *     chunk.  ciera: the r-th changed block owns slots rB..rB+B-1.
 *
 * Conventions for every entry point:
 *  - d_* arguments are device pointers on the current HIP device, 16-byte
 *    aligned, owned and allocated by the caller.  The library never
 *    allocates, frees or synchronises (except ciera_read_error).  Buffers
 *    must not alias.
 *  - BF16 data is passed as its 16-bit patterns (n values = 2n bytes).
 *  - Calls are asynchronous on `stream`: they return once the kernels are
 *    enqueued.  Argument errors are reported synchronously, before any
 *    launch, and nothing is enqueued then.  Errors found on the device (a
 *    malformed stream in decode) are written to the workspace; read them
 *    with ciera_read_error.
 *  - The workspace is caller-owned scratch of at least the size the
 *    *_workspace_size query returns.  Its contents need no initialisation
 *    and are meaningless between calls, except for the error words that
 *    ciera_read_error reads.  Calls that share a workspace must be ordered
 *    (same stream, or synchronised); distinct workspaces may be used
 *    concurrently on different streams.
 *  - n <= 2^40.  n = 0 is valid.  B is a power of two, 64 <= B <= 65536.
 *  - Within an encode, workgroups wait on each other only through bounded
 *    waits on lower-numbered workgroups (which the GPU dispatches first), so
 *    an encode completes while other kernels share the GPU.  A wait that
 *    runs out of its bound (seconds of polling) makes ciera_read_error
 *    report CIERA_ERR_INTERNAL.  The stream is then not valid and must not
 *    be sent; the 3-bit encodes with a derived window (zip3_encode,
 *    ciera_encode, ciera_encode_hashed, *_encode_ex) also set *d_out_size
 *    to 0 and clear the header's first 8 bytes.  The sender's cache (or
 *    hash cache) may then hold the new exponents (hashes) of some blocks
 *    and the previous ones of others, so the caches of sender and receivers
 *    are out of step: zero the sender's cache and every receiver's cache
 *    before the next iteration (a full resend).
 */
#ifndef CIERA_H
#define CIERA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int ciera_status;
#define CIERA_OK 0
#define CIERA_ERR_ARG 1       /* null or misaligned pointer, n too large, bad B or E0 override */
#define CIERA_ERR_CAPACITY 2  /* out_capacity below the *_max_encoded_size bound */
#define CIERA_ERR_WORKSPACE 3 /* ws_bytes below the *_workspace_size bound */
#define CIERA_ERR_HIP 4       /* a HIP launch or runtime call failed */
#define CIERA_ERR_FORMAT 5    /* decode: the stream is malformed or does not match n / B / mode */
#define CIERA_ERR_INTERNAL 6  /* encode: a wait on another workgroup gave up (see below) */

#define CIERA_CHUNK 65536u

/* Largest stream zip3_encode can write for n values (every value an escape):
 * about 2.375 n bytes plus headers.  Pass at least this as out_capacity. */
uint64_t zip3_max_encoded_size(uint64_t n);
/* Same for ciera_encode with block size B (every block changed).  Returns 0
 * for an invalid B. */
uint64_t ciera_max_encoded_size(uint64_t n, uint32_t B);
/* Workspace bytes needed by zip3_encode and zip3_decode for n values. */
uint64_t zip3_workspace_size(uint64_t n);
/* Workspace bytes needed by ciera_encode and ciera_decode for n values and
 * block size B (0 for an invalid B). */
uint64_t ciera_workspace_size(uint64_t n, uint32_t B);

/* zip3_encode: code every exponent of x (ZipCCL digest, section 3.1).
 *   d_x        in   n BF16 patterns (u16), 16-byte aligned
 *   d_out      out  the stream; out_capacity >= zip3_max_encoded_size(n)
 *   d_ws       tmp  ws_bytes >= zip3_workspace_size(n)
 *   d_out_size out  one u64 on the device: the stream's length in bytes
 *                   (also in header bytes 32..39).  Read it after syncing.
 * Errors: CIERA_ERR_ARG, _CAPACITY, _WORKSPACE, _HIP (synchronous). */
ciera_status zip3_encode(const void* d_x, uint64_t n, void* d_out, uint64_t out_capacity,
                         void* d_ws, uint64_t ws_bytes, uint64_t* d_out_size,
                         hipStream_t stream);

/* zip3_decode: inverse of zip3_encode.
 *   d_in   in   the stream, in_size bytes (at least its total_bytes)
 *   d_y    out  n BF16 patterns, bit-identical to the encoded input
 *   d_ws   tmp  ws_bytes >= zip3_workspace_size(n)
 * A stream whose header, table or section sizes do not match n and the
 * layout is rejected on the device: the kernels read nothing outside
 * [d_in, d_in + in_size), leave d_y unspecified, and ciera_read_error then
 * returns CIERA_ERR_FORMAT. */
ciera_status zip3_decode(const void* d_in, uint64_t in_size, void* d_y, uint64_t n,
                         void* d_ws, uint64_t ws_bytes, hipStream_t stream);

/* ciera_encode: exponent reuse across iterations plus the 3-bit code for the
 * changed blocks (CIERA page, sections 3.1-3.2; ZipCCL digest, section 3.1).
 *   d_x         in      n BF16 patterns of this iteration
 *   B           in      block size
 *   d_prev_exp  in/out  sender exponent cache, n bytes: the exponent fields
 *                       of the previous iteration's tensor (all zero before
 *                       the first).  On return it holds x's exponents.
 *   d_out, out_capacity >= ciera_max_encoded_size(n, B), d_ws, ws_bytes >=
 *   ciera_workspace_size(n, B), d_out_size: as for zip3_encode.
 * The window E0 comes from the standard deviation of all finite values of
 * x, not only of the changed blocks. */
ciera_status ciera_encode(const void* d_x, uint64_t n, uint32_t B, uint8_t* d_prev_exp,
                          void* d_out, uint64_t out_capacity, void* d_ws, uint64_t ws_bytes,
                          uint64_t* d_out_size, hipStream_t stream);

/* ciera_encode_hashed: ciera_encode with the sender state of the CIERA page
 * (section 3.1): per block a 128-bit hash of its exponents made of two
 * independent 64-bit SplitMix64 hashes, in place of the n-byte exponent
 * cache, so encode reads 16 bytes per block instead of one byte per value.
 * A block counts as unchanged only when both hashes equal the stored ones.
 * The stream is the one ciera_encode writes from an exponent cache holding
 * the previous exponents, unless a changed block's two hashes both collide
 * with the stored ones (about 2^-128 per comparison); the receiver side is
 * ciera_decode with its exponent cache, unchanged.
 *   d_hash_cache  in/out  ciera_hash_cache_size(n, B) bytes, 16-byte aligned:
 *                 per block two u64, the hashes of the exponents last sent.
 *                 Zero-filled before the first iteration: (0, 0) is the hash
 *                 of all-zero exponents, so the first stream equals
 *                 ciera_encode's from a zeroed exponent cache.  Changed
 *                 blocks get their new hashes.
 * Block hash: block b's exponent fields, 8 at a time, form little-endian u64
 * words w_k (the last word of a short block zero-filled); hash j is the sum
 * mod 2^64, over the words that are not zero, of SplitMix64's output function
 * at w_k + s_j + (k + 1) g_j, i.e. the (k+1)-th output of a SplitMix64
 * generator with seed w_k + s_j and increment g_j; (s_0, g_0) =
 * (0, 0x9E3779B97F4A7C15), (s_1, g_1) = (0x243F6A8885A308D3,
 * 0xD1B54A32D192ED03).
 * Other arguments, the workspace and errors as ciera_encode; CIERA_ERR_ARG
 * also for a misaligned d_hash_cache, or a null one with n > 0. */
ciera_status ciera_encode_hashed(const void* d_x, uint64_t n, uint32_t B, void* d_hash_cache, void* d_out,
                                 uint64_t out_capacity, void* d_ws, uint64_t ws_bytes, uint64_t* d_out_size,
                                 hipStream_t stream);

/* Bytes of the hash sender's cache: 16 per block of B values (0 for an
 * invalid B or n above 2^40). */
uint64_t ciera_hash_cache_size(uint64_t n, uint32_t B);

/* rANS modes (mode byte 2: zip3 + rANS, 3: ciera + rANS).  The coded
 * exponents (every value's in zip3 mode, the changed blocks' in ciera mode)
 * are entropy coded with range ANS instead of the 3-bit window code, as the
 * CIERA page ANS-codes the changed exponents (section 3.1; the page names
 * no ANS parameters, so this coder and its format are ours):
 *   - per chunk, one frequency table: the histogram of all the chunk's
 *     coded exponent fields normalised to 4096: with d distinct symbols
 *     among m, f = max(1, floor(h (4096 - d) / m)) for each present
 *     symbol, the remainder to the most frequent one (the lowest on ties);
 *   - per part (16384 values of a chunk) the symbols are its coded exponent
 *     fields in value order, coded with the chunk's table by 64 interleaved
 *     rANS states, symbol i to state i mod 64, 32-bit states in
 *     [2^16, 2^32) starting at 2^16, 16-bit renormalisation words;
 *   - chunk payload: u8 lo, u8 hi, u16 0, u16 w_0 .. w_3 (the 16-bit words
 *     of each part's stream; 0 for a part without coded symbols), u16
 *     frequencies of symbols lo..hi, then the part streams in part order: a
 *     part's 64 final states (low, high half), then the words each step
 *     emitted, steps in decode order, states ascending within a step;
 *   - stream (version 2): the 128-byte header (E0 byte 0; bytes 48..55 the
 *     number of coded symbols), a table of nchunks + 1 u64 absolute payload
 *     offsets (the last equals total_bytes) zero-padded to 128, the
 *     sign+mantissa bytes of all n values zero-padded to 128, in ciera mode
 *     one 128-byte bitmap per chunk, then the chunk payloads, each
 *     zero-padded to 128.
 * Arguments, caches, ownership and errors as the 3-bit entry points; the
 * workspace is rans_workspace_size(n, B) bytes for encode (it holds a
 * payload scratch slot per chunk) and *_workspace_size(n) for decode; the
 * output capacity rans_max_encoded_size(n, B).  As for the 3-bit streams,
 * a decoder's in_size is the buffer's size: at least the stream's
 * total_bytes, whose bytes alone are read.  Encode's workgroups wait on
 * earlier ones for their stream offsets (bounded waits, reported as
 * CIERA_ERR_INTERNAL).  Decode checks the header, the chunk table, every
 * payload's word counts, length and padding, that the frequencies sum to
 * 4096, that every word is used and every state ends at 2^16 (else
 * CIERA_ERR_FORMAT; the output and the receiver cache are then undefined). */
uint64_t rans_max_encoded_size(uint64_t n, uint32_t B);
uint64_t rans_workspace_size(uint64_t n, uint32_t B);
ciera_status zip3_encode_rans(const void* d_x, uint64_t n, void* d_out, uint64_t out_capacity, void* d_ws,
                              uint64_t ws_bytes, uint64_t* d_out_size, hipStream_t stream);
ciera_status zip3_decode_rans(const void* d_in, uint64_t in_size, void* d_y, uint64_t n, void* d_ws,
                              uint64_t ws_bytes, hipStream_t stream);
ciera_status ciera_encode_rans(const void* d_x, uint64_t n, uint32_t B, uint8_t* d_prev_exp, void* d_out,
                               uint64_t out_capacity, void* d_ws, uint64_t ws_bytes, uint64_t* d_out_size,
                               hipStream_t stream);
ciera_status ciera_decode_rans(const void* d_in, uint64_t in_size, void* d_y, uint64_t n, uint32_t B,
                               uint8_t* d_prev_exp, void* d_ws, uint64_t ws_bytes, hipStream_t stream);

/* ciera_decode: rebuild x from the stream and the receiver's cache.
 *   d_prev_exp  in/out  receiver exponent cache, n bytes, holding the
 *                       previous iteration's exponents (all zero before the
 *                       first); blocks the bitmap marks unchanged take their
 *                       exponents from it.  On return it holds x's exponents.
 * Other arguments and error behaviour as zip3_decode; B must equal the
 * stream's B. */
ciera_status ciera_decode(const void* d_in, uint64_t in_size, void* d_y, uint64_t n, uint32_t B,
                          uint8_t* d_prev_exp, void* d_ws, uint64_t ws_bytes, hipStream_t stream);

/* zip3_decode_batch, ciera_decode_batch: k streams of the same n (and B)
 * decoded in one launch, e.g. the peer shards a rank receives in a sharded
 * all-gather: the CIERA page's receivers decompress each peer's message
 * against that peer's receiver cache (section 3.1; the pipelining of section
 * 3.3 puts this decompression on the critical path).  Stream i is decoded
 * exactly as zip3_decode / ciera_decode would decode it alone.
 *   k           1..CIERA_DECODE_BATCH_MAX
 *   d_in[i], in_size[i]  stream i and its buffer's size (as in_size of the
 *                        single decode); host arrays of k entries, read
 *                        during the call
 *   d_y[i]      output i, n u16, 16-B aligned; the k outputs must not overlap
 *   d_prev_exp[i]  (ciera) receiver cache of stream i's sender, n bytes,
 *                  in/out as in ciera_decode; the k caches must not overlap
 *   d_ws        workspace of decode_batch_workspace_size(n, k) bytes: one
 *               status word per workgroup of all k streams
 * Argument errors (k out of range, k * n above 2^40, a null or misaligned
 * pointer, a small workspace) return before any launch.  A malformed stream
 * makes ciera_read_error report CIERA_ERR_FORMAT (without saying which
 * stream); that stream's output and cache are then unspecified, the other
 * streams are decoded in full. */
#define CIERA_DECODE_BATCH_MAX 16u
uint64_t decode_batch_workspace_size(uint64_t n, uint32_t k);
ciera_status zip3_decode_batch(uint32_t k, const void* const* d_in, const uint64_t* in_size, void* const* d_y,
                               uint64_t n, void* d_ws, uint64_t ws_bytes, hipStream_t stream);
ciera_status ciera_decode_batch(uint32_t k, const void* const* d_in, const uint64_t* in_size, void* const* d_y,
                                uint64_t n, uint32_t B, uint8_t* const* d_prev_exp, void* d_ws, uint64_t ws_bytes,
                                hipStream_t stream);

/* Synchronise `stream` and return the device-side status of the last call
 * that used d_ws: CIERA_OK, CIERA_ERR_FORMAT (decode saw a malformed
 * stream), CIERA_ERR_INTERNAL, or CIERA_ERR_HIP if the copy fails. */
ciera_status ciera_read_error(const void* d_ws, hipStream_t stream);

/* zip3_encode_e0: zip3 encode with the window base read from device memory
 * instead of derived from the standard deviation, so that x is read once
 * (no variance pass).  The digest's window rule (section 3.1) sets E0 from
 * the tensor's sigma; a caller that takes E0 from an earlier tensor, e.g.
 * byte 7 of the previous iteration's stream header, trades a possibly less
 * central window for one read of x instead of two.
 *   d_e0  in  device pointer to one byte, the window base (0..249); read on
 *             the device when the encode runs, so it may be produced by
 *             earlier work on `stream`.  A value above 249 makes the call
 *             write only the stream's first 8 bytes, whose E0 byte (byte 7)
 *             keeps that value, so that a decoder rejects the stream and a
 *             next encode that takes its window base from byte 7 is refused
 *             too; *d_out_size becomes 0 and ciera_read_error reports
 *             CIERA_ERR_ARG.
 * Other arguments, sizes and the workspace as zip3_encode, except that n is
 * limited to 2^39 (CIERA_ERR_ARG above); the stream equals zip3_encode_ex's
 * with e0_override = *d_e0.  Within the call, workgroups
 * wait on each other through the workspace (bounded waits; a wait that does
 * not end is reported as CIERA_ERR_INTERNAL by ciera_read_error).  A tensor
 * of at most 16 chunks (2^20 values; its 2 MiB stay in the GPU's last-level
 * cache) is encoded by the two launches of zip3_encode with the given window
 * base instead: x is read twice there, and no workgroup waits. */
ciera_status zip3_encode_e0(const void* d_x, uint64_t n, const uint8_t* d_e0, void* d_out, uint64_t out_capacity,
                            void* d_ws, uint64_t ws_bytes, uint64_t* d_out_size, hipStream_t stream);

/* ciera_encode_e0: ciera_encode with the window base read from device memory
 * (d_e0, as in zip3_encode_e0), so that x and the sender cache are read
 * once: each part compares its exponents with the cache, rewrites the
 * bytes that differ and codes its changed blocks in the same pass.  The
 * CIERA page keeps the exponents of unchanged blocks out of the message
 * (section 3.1); the window rule of the ZipCCL digest (section 3.1) sets
 * E0 from the tensor's sigma, here the caller's choice (e.g. byte 7 of the
 * previous iteration's stream header).  Arguments, caches, sizes and the
 * workspace as ciera_encode (workspace ciera_workspace_size(n, B)), except
 * that n is limited to 2^39 (CIERA_ERR_ARG above); the stream and the cache
 * equal ciera_encode_ex's with e0_override = *d_e0.  A *d_e0 above 249 leaves
 * the cache as it was and the stream and *d_out_size as zip3_encode_e0 does
 * (CIERA_ERR_ARG).  Workgroups wait on each other through the
 * workspace as in zip3_encode_e0, and a tensor of at most 16 chunks is
 * encoded by ciera_encode's two launches with the given window base, as
 * there. */
ciera_status ciera_encode_e0(const void* d_x, uint64_t n, uint32_t B, uint8_t* d_prev_exp, const uint8_t* d_e0,
                             void* d_out, uint64_t out_capacity, void* d_ws, uint64_t ws_bytes, uint64_t* d_out_size,
                             hipStream_t stream);

/* zip3_encode_spec, ciera_encode_spec: zip3_encode / ciera_encode with the
 * same stream, cache and *d_out_size for every input, but x (and the sender
 * cache) read once when a hint names the right window base.  The window rule
 * of the ZipCCL digest (section 3.1) takes E0 from the current tensor's
 * sigma; sigma moves little from one training iteration to the next, so the
 * previous iteration's E0 (byte 7 of its stream) is usually the same.  The
 * call writes the stream in one pass with the hinted window while it adds
 * the variance sums, then checks on the device that the variance gives that
 * window; if not (or the hint is above 249, or a wait between workgroups did
 * not end), it encodes again with the two-pass kernels, taking the changed
 * blocks it recorded in the first pass (CIERA page, section 3.1), so the
 * result is still ciera_encode's.
 *   d_hint  in  device pointer to one byte, the hinted window base, read
 *               when the encode runs (it may be the previous stream's byte 7
 *               in the same output buffer)
 * Other arguments, sizes, workspace (zip3/ciera_workspace_size) and errors
 * as zip3_encode / ciera_encode.  A tensor of at most 16 chunks, or of more
 * than 2^39 values, is encoded by zip3_encode / ciera_encode without the
 * hint.  A right hint costs the single-read encode plus three small kernels
 * and three launches that return at once; a wrong one the single-read pass
 * plus the two-pass encode.  If a wait of the two-pass kernels then does not
 * end either, the call ends as ciera_encode does after CIERA_ERR_INTERNAL
 * (*d_out_size 0, the header's first word cleared; the sender cache holds
 * x's exponents, so both caches are zeroed before the next iteration). */
ciera_status zip3_encode_spec(const void* d_x, uint64_t n, const uint8_t* d_hint, void* d_out, uint64_t out_capacity,
                              void* d_ws, uint64_t ws_bytes, uint64_t* d_out_size, hipStream_t stream);
ciera_status ciera_encode_spec(const void* d_x, uint64_t n, uint32_t B, uint8_t* d_prev_exp, const uint8_t* d_hint,
                               void* d_out, uint64_t out_capacity, void* d_ws, uint64_t ws_bytes, uint64_t* d_out_size,
                               hipStream_t stream);

/* Kernel timing, a profiling aid (not part of the codec).  events holds
 * n_pairs (start, stop) pairs of hipEvent_t handles, created with timing
 * enabled and owned by the caller.  The next n_pairs kernel launches made by
 * the calling host thread through this library (any entry point: the
 * 3-bit encode launches four kernels, or two for a tensor of at most 16
 * chunks, whose planning the write kernel does itself, unless plan_groups
 * forces the planner; its decode one; the single-read encode two; the rANS
 * encode three and its decode one; the speculative encode seven on a tensor
 * of more than 16 chunks, whatever the hint; the batch decode one) each take
 * the next pair, which the HIP runtime records at that kernel's start and end
 * (hipExtLaunchKernel);
 * hipEventElapsedTime then gives the kernel's own duration.  The handles are
 * copied; a later call replaces the queue, n_pairs = 0 clears it.  Returns
 * CIERA_ERR_ARG for a null array or handle. */
ciera_status ciera_time_kernels(void* const* events, uint32_t n_pairs);

/* ciera_encode_noalloc: ciera_encode for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same kernels, stream, cache update
 * and window, with the workspace taken from a 6 MiB array that the library
 * holds in device memory (one per GPU it runs on, kept until the process
 * ends) instead of a caller's buffer.  The call allocates and frees
 * nothing; its first call on a device looks up that device's array.
 *   d_x, n, B, d_prev_exp, d_out, out_capacity, d_out_size: as ciera_encode.
 *   n <= CIERA_NOALLOC_MAX_N (2^27 values); a larger n returns
 *   CIERA_ERR_WORKSPACE before anything is enqueued.
 * Every call on one GPU uses that GPU's one array: calls that overlap on a
 * GPU (two streams, or two host threads) race and corrupt each other's
 * streams; order them.  The kernels clear what they need, so the array's
 * contents from an earlier call do not matter.  There is no workspace for
 * ciera_read_error: a wait that gave up shows as *d_out_size == 0 once the
 * stream has completed (the header's state as after CIERA_ERR_INTERNAL). */
#define CIERA_NOALLOC_MAX_N (1ull << 27)
ciera_status ciera_encode_noalloc(const void* d_x, uint64_t n, uint32_t B, uint8_t* d_prev_exp, void* d_out,
                                  uint64_t out_capacity, uint64_t* d_out_size, hipStream_t stream);

/* Test hook: the number of polls after which the next calls' waits on
 * other workgroups give up (CIERA_ERR_INTERNAL); 0 restores the default
 * (2^22).  Returns the previous value.  Tests lower it to drive the failure
 * path from the host with every kernel still ending normally.  Applies to
 * calls made after it, from any thread. */
uint32_t ciera_set_wait_limit(uint32_t polls);

/* Human-readable name of a status code (static storage). */
const char* ciera_status_string(ciera_status status);

/* Same as zip3_encode / ciera_encode with the window base forced to
 * e0_override (0..249); -1 derives it from the standard deviation as the
 * plain entry points do.  For tests that pin the layout at a given window
 * and for callers that reuse the previous iteration's window.
 *   plan_groups  0 for the default; otherwise the planning step (which
 *                reduces the variance sums and lays out the chunk table)
 *                runs on at most this many workgroups, each taking more
 *                chunks.  The stream does not depend on it; tests use it to
 *                reach the long-range paths of the planner with small inputs.
 *                The window base may differ only where the variance lies
 *                within rounding of a threshold (the sums' order changes). */
ciera_status zip3_encode_ex(const void* d_x, uint64_t n, void* d_out, uint64_t out_capacity,
                            void* d_ws, uint64_t ws_bytes, uint64_t* d_out_size, int e0_override,
                            uint32_t plan_groups, hipStream_t stream);
ciera_status ciera_encode_ex(const void* d_x, uint64_t n, uint32_t B, uint8_t* d_prev_exp,
                             void* d_out, uint64_t out_capacity, void* d_ws, uint64_t ws_bytes,
                             uint64_t* d_out_size, int e0_override, uint32_t plan_groups,
                             hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* CIERA_H */
