/*
 * w4a16.h - C ABI of libw4a16: the decode-step matrix-vector product over
 * 4-bit group-quantised weights and 16-bit activations (W4A16) on gfx950.
 *
 * Sources. The core-modules page (section 5.1, packer: quantisation) places
 * edge decode in the 4-bit-weight / 16-bit-activation regime; its runtime
 * table (section 5.2) names the K-quant Q4_K_M family; the Magnitude page
 * (section 3.4, thread control) and the core-modules page (section 5.4,
 * loading strategies) frame decode as memory-bandwidth bound, which is why the
 * kernel streams each weight exactly once. Section 5.2's list of runtime
 * traits (static shapes, an allocation-free decode loop, a plain tensor
 * descriptor behind a backend table) sets the conventions below: plain
 * pointers and sizes, caller-owned buffers, no allocation, no
 * synchronisation. Section 5.7's contract table (a runtime refuses a model
 * whose format it does not cover) is why every argument error is reported
 * as a status instead of being run.
 *
 * Weight format (the plain reading of "group scale and min"; the pages never
 * spell the format out):
 *   codes  uint8 [N][K/2]  two unsigned 4-bit codes per byte, row n = output
 *                          feature n; the LOW nibble of byte j is k = 2j, the
 *                          HIGH nibble is k = 2j + 1.
 *   scale  binary16 [N][K/32], min binary16 [N][K/32]: one pair per group of
 *                          32 consecutive k of one row.
 *   w_hat[n][k] = scale[n][k/32] * q[n][k] + min[n][k/32]
 *   y[m][n]     = sum_k w_hat[n][k] * x[m][k]      (x binary16 [M][K], y fp32)
 *
 * Packed layout (what w4a16_pack writes and w4a16_gemv reads):
 *   G  = K / 32 groups per row, T = ceil(N / 4) row tiles. Every blob of
 *   every codec starts with the same 256-byte header, then its regions at the
 *   offsets given below relative to byte H = 256:
 *   [0, 256)             header, little endian: uint32 magic
 *                        W4A16_BLOB_MAGIC at byte 0, uint16
 *                        W4A16_LAYOUT_VERSION at 4, uint16 codec at 6
 *                        (W4A16_CODEC_*; 0 for w4a16_pack), int32 N at 8,
 *                        int32 K at 12, uint64 blob bytes at 16, zeros up to
 *                        byte 256. The kernels compare bytes 0..15 with the
 *                        call's codec, N and K (see w4a16_gemv).
 *   H + [0, N*K/2)       codes: row-major [N][G] chunks of 16 bytes; chunk
 *                        (n, g) holds k = 32g .. 32g+31. Inside a chunk, the
 *                        little-endian 32-bit word d (bytes 4d..4d+3) holds
 *                        k = 32g + 8d + i, i = 0..7, with nibble slot p
 *                        (bits 4p..4p+3) holding i = 2p for p < 4 and
 *                        i = 2(p-4)+1 for p >= 4: the four even i in the low
 *                        half-word, the four odd i in the high half-word,
 *                        each in increasing order.
 *   H + [S, S + T*G*16)  S = N*K/2 rounded up to a multiple of 256. Scale/min
 *                        tiles: [T][G] entries of 16 bytes; entry (t, g) holds
 *                        rows 4t .. 4t+3, row r in bytes 4r..4r+3 as
 *                        (binary16 scale, binary16 min), little endian. Rows
 *                        at or beyond N are zero.
 *   Total size: w4a16_packed_bytes(N, K) = 256 + S + T*G*16.
 *
 * Status codes are returned, never raised; nothing aborts.
 */
#ifndef W4A16_H
#define W4A16_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum w4a16_status {
  W4A16_OK = 0,
  W4A16_ERR_NULL = 1,     /* a required pointer is NULL */
  W4A16_ERR_SHAPE = 2,    /* M, N or K outside the supported range */
  W4A16_ERR_ALIGN = 3,    /* a pointer breaks its alignment rule */
  W4A16_ERR_SIZE = 4,     /* an output buffer is smaller than required */
  W4A16_ERR_OVERLAP = 5,  /* y overlaps x or the packed weights */
  W4A16_ERR_HIP = 6,      /* the HIP runtime reported an error */
  W4A16_ERR_FORMAT = 7,   /* unknown codec, a code outside its codec's range, or a
                             blob header that does not match the call */
  W4A16_ERR_WAIT = 8      /* a chain launch's ordering wait gave up: its results are invalid */
} w4a16_status;

/* First four bytes of every packed weight blob ("W416" in ASCII). */
#define W4A16_BLOB_MAGIC 0x36313457u
/* Version of the packed layouts, stored in every blob header. */
#define W4A16_LAYOUT_VERSION 6
/* Bytes of the header that starts every packed weight blob. */
#define W4A16_BLOB_HEADER_BYTES 256

/* Version of this ABI (equal to W4A16_LAYOUT_VERSION); bumped on any change. */
int32_t w4a16_abi_version(void);

/* Largest K accepted by w4a16_gemv for a given M (0 if M is outside 1..8). */
int32_t w4a16_max_k(int32_t M);

/*
 * Bytes of the packed blob for an N x K weight matrix (see "Packed layout"):
 * the size of the one-off re-layout the packer of the core-modules page
 * (section 5.1, quantisation) produces, which the memory manager's weight
 * budget (section 5.4) has to hold, about 0.63 bytes per weight.
 * Returns 0 if N < 1, K < 32, K % 32 != 0, or N * K / 32 does not fit the
 * kernels' 31-bit chunk index.
 */
size_t w4a16_packed_bytes(int32_t N, int32_t K);

/*
 * w4a16_blob_check - host only: is `blob` (a host copy of at least its first
 * 256 bytes; `bytes` = how many bytes the caller holds or will upload) a
 * packed blob of this layout version for (codec, N, K)? The format refusal
 * of the core-modules page's contract table (section 5.7: a runtime refuses
 * a model file it cannot run), for loaders to call before uploading.
 * Returns W4A16_OK; W4A16_ERR_NULL for a NULL blob; W4A16_ERR_SHAPE for an
 * unknown codec or bad N/K; W4A16_ERR_FORMAT if the magic, version, codec,
 * N, K or recorded size differ; W4A16_ERR_SIZE if bytes is below the blob's
 * size (only the first 256 bytes are read).
 */
w4a16_status w4a16_blob_check(const void* blob, size_t bytes, int32_t codec, int32_t N, int32_t K);

/*
 * w4a16_blob_mismatches - launches on the current device whose packed blob's
 * header did not match their call (codec, N, K or layout version), counted
 * since the previous call of this function, which resets the count. Those
 * launches wrote nothing to y. Synchronises the current device first.
 * Errors: NULL -> W4A16_ERR_NULL; a HIP failure -> W4A16_ERR_HIP.
 */
w4a16_status w4a16_blob_mismatches(uint32_t* count);

/*
 * w4a16_pack - host-side repacker (init time; not on the per-token path).
 * The packer's quantise-then-lay-out step of the core-modules page (section
 * 5.1), done once so the run-time kernel only ever streams.
 *
 *   codes  host uint8 [N][K/2], layout as in "Weight format"   (read only)
 *   scale  host binary16 bits [N][K/32]                         (read only)
 *   min    host binary16 bits [N][K/32]                         (read only)
 *   out    host buffer of at least w4a16_packed_bytes(N, K) bytes, owned
 *          by the caller; written completely (header, then regions; padding
 *          is zeroed).
 * The caller then copies `out` to device memory, 256-byte aligned.
 * Uses worker threads for large inputs; touches no GPU.
 * Errors: NULL pointer -> W4A16_ERR_NULL; bad N/K -> W4A16_ERR_SHAPE;
 * out_bytes too small -> W4A16_ERR_SIZE (nothing written).
 */
w4a16_status w4a16_pack(const uint8_t* codes, const uint16_t* scale, const uint16_t* min,
                        int32_t N, int32_t K, void* out, size_t out_bytes);

/*
 * w4a16_gemv - y[M][N] = x[M][K] * w_hat^T, one decode-step product (the
 * per-token GEMV of every fused linear layer, core-modules page section 5.1's
 * fused query/key/value and gate/up rewrites; M > 1 rows are a speculative
 * verify batch, section 5.6).
 *
 *   x       device binary16 [M][K], row-major, 16-byte aligned (read only)
 *   packed  device blob written by w4a16_pack for this N and K, 256-byte
 *           aligned (read only)
 *   y       device fp32 [M][N], row-major, 4-byte aligned; overwritten (no
 *           accumulation into prior contents)
 *   M       activation rows, 1..8
 *   N       output features, >= 1
 *   K       input features, multiple of 32, 32 <= K <= w4a16_max_k(M)
 *   stream  hipStream_t to enqueue on (NULL = the device's null stream)
 *
 * All buffers are owned by the caller and must live until the work completes.
 * The call only enqueues: it never allocates, frees or synchronises. Results
 * are bitwise repeatable for the same inputs on the same device.
 * Errors (checked on the host before anything is enqueued): NULL pointer ->
 * W4A16_ERR_NULL; M, N or K out of range -> W4A16_ERR_SHAPE; misaligned
 * pointer -> W4A16_ERR_ALIGN; y's byte range intersecting x's or the packed
 * blob's -> W4A16_ERR_OVERLAP; a launch the HIP runtime rejects ->
 * W4A16_ERR_HIP. The blob header is checked on the device, by one scalar load
 * issued beside the first weight loads: if its magic, layout version, codec,
 * N or K differ from this call's, the kernel writes nothing to y and counts
 * the launch in w4a16_blob_mismatches. The weight loads are not held back by
 * that check, so a blob shorter than w4a16_packed_bytes(N, K) is still read
 * out of bounds: such faults are not detectable here and surface at the
 * caller's next synchronisation (w4a16_blob_check refuses such a blob on the
 * host before upload).
 */
w4a16_status w4a16_gemv(const void* x, const void* packed, float* y,
                        int32_t M, int32_t N, int32_t K, void* stream);

/*
 * w4a16_launch_shape - how w4a16_gemv would run an (M, N, K) product, for
 * profilers and benches that attribute kernel time to launches. Pure host
 * logic: touches no GPU.
 *   out[0] = groups of 32 k per lane (the kernel's template parameter),
 *   out[1] = waves per workgroup, out[2] = passes over K.
 * The kernel symbol is gemv_kernel<M, out[0]>.
 * Errors: out NULL -> W4A16_ERR_NULL; shape outside w4a16_gemv's range ->
 * W4A16_ERR_SHAPE (out untouched).
 */
w4a16_status w4a16_launch_shape(int32_t M, int32_t N, int32_t K, int32_t out[3]);

/*
 * w4a16_gemv_timed - w4a16_gemv, with the kernel's own start and end times
 * recorded into two caller-owned HIP events (hipEvent_t, created with timing
 * enabled, e.g. by hipEventCreate): their elapsed time is the kernel's
 * execution alone, the duration a profiler reports for it, without the
 * launch latency that events recorded around the call would also include.
 * Arguments, results and errors are those of w4a16_gemv; either event NULL
 * -> W4A16_ERR_NULL.
 */
w4a16_status w4a16_gemv_timed(const void* x, const void* packed, float* y, int32_t M, int32_t N, int32_t K,
                              void* stream, void* start_event, void* stop_event);

/*
 * Decode-step chain: the GEMVs of a whole decode step in ONE kernel launch.
 *
 * The runtime traits of the core-modules page (section 5.2: a tight decode
 * loop, static shapes fixed before the loop) and its scheduler enhancements
 * (section 5.3: prefetch the next matrix product's weights while other work
 * runs) motivate it: a decode step runs the same list of products every
 * token, each product's input usually depends on the previous one's output,
 * and on an MI355X a kernel boundary costs about as much as streaming 10 MB
 * of weights. The chain runs the list in order inside one persistent launch;
 * before each product it waits (on a device-side counter) until every
 * earlier product's results are written, and while it waits the next
 * product's weights are already being streamed, since weights never depend
 * on earlier results.
 */
typedef struct w4a16_chain_entry {
  const void* x;       /* device binary16 [M][K], 16-byte aligned */
  const void* packed;  /* device blob from w4a16_pack for (N, K), 256-byte aligned */
  float* y;            /* device fp32 [M][N], 4-byte aligned, overwritten */
  int32_t N;           /* output features, >= 1 */
  int32_t K;           /* input features, multiple of 32, 32 <= K <= w4a16_max_k(M) */
} w4a16_chain_entry;

/* Bytes of the device workspace of w4a16_gemv_chain. */
#define W4A16_CHAIN_WORKSPACE_BYTES 69632
/* Byte offset in that workspace of the uint32 error word, a set of the bits
 * below, raised by a chain launch and never cleared by one. Any bit set:
 * results of that call are invalid; zero-fill the workspace again before the
 * next call. */
#define W4A16_CHAIN_ERROR_OFFSET 256
#define W4A16_CHAIN_ERR_WAIT 1u  /* an ordering wait gave up */
#define W4A16_CHAIN_ERR_PLAN 2u  /* the plan's header does not match (count, M): nothing was written */
#define W4A16_CHAIN_ERR_BLOB 4u  /* an entry's blob header does not match its (N, K): no y was written */

/* Most entries of one chain plan. */
#define W4A16_CHAIN_MAX_ENTRIES 1048576

/* Bytes of the plan for `count` entries (0 if count < 1 or
 * count > W4A16_CHAIN_MAX_ENTRIES). */
size_t w4a16_chain_plan_bytes(int32_t count);

/*
 * w4a16_chain_plan - host only, init time: validate a list of products that
 * share the activation-row count M and write the device-ready plan into the
 * caller's host buffer `plan` (at least w4a16_chain_plan_bytes(count) bytes).
 * The caller copies the plan to device memory (16-byte aligned) and keeps it
 * for as many steps as the buffers it names stay put.
 * Rules, each checked here: every entry is a valid w4a16_gemv call for M
 * (shape, alignment, y disjoint from its own x and packed blob); no packed
 * blob intersects any entry's y (weights are read ahead of the ordering
 * point). An entry's x MAY overlap an earlier entry's y: that is the
 * dependency the chain honours.
 * Errors: NULL -> W4A16_ERR_NULL; bad count/M/shape -> W4A16_ERR_SHAPE;
 * alignment -> W4A16_ERR_ALIGN; plan_bytes too small -> W4A16_ERR_SIZE;
 * overlap -> W4A16_ERR_OVERLAP. Nothing is written on error. Touches no GPU.
 */
w4a16_status w4a16_chain_plan(const w4a16_chain_entry* entries, int32_t count, int32_t M, void* plan,
                              size_t plan_bytes);

/*
 * w4a16_gemv_chain - enqueue the planned products on `stream` as one kernel.
 * The results are those of w4a16_gemv on each entry in order, up to the fp32
 * summation order (within the same tolerance, and bitwise repeatable from
 * run to run); entry i observes every y written by entries 0..i-1.
 *   plan       device copy of a plan from w4a16_chain_plan(..., count, M, ...)
 *   workspace  device buffer of workspace_bytes >= W4A16_CHAIN_WORKSPACE_BYTES,
 *              16-byte aligned, zero-filled by the caller once before its first use;
 *              every call leaves its counters at zero again. The uint32 at
 *              W4A16_CHAIN_ERROR_OFFSET becomes nonzero if an ordering wait
 *              ever gave up (waits bound their spin so a starved launch
 *              cannot hang the GPU), the plan or a blob header did not
 *              match; results of such a call are invalid. Calls that share
 *              a workspace must not run concurrently.
 * The plan and workspace are owned by the caller. The call only enqueues.
 * The launch keeps all of its workgroups resident (grid sized from the
 * occupancy of the kernel); other work running concurrently on the device
 * can delay it but not deadlock it.
 * Errors (host side): NULL -> W4A16_ERR_NULL; count outside
 * 1..W4A16_CHAIN_MAX_ENTRIES or M outside 1..8 ->
 * W4A16_ERR_SHAPE; misaligned plan or workspace -> W4A16_ERR_ALIGN;
 * workspace_bytes too small -> W4A16_ERR_SIZE; launch rejected ->
 * W4A16_ERR_HIP. A plan whose header does not match (count, M) is detected
 * on the device: the kernel then writes nothing and raises
 * W4A16_CHAIN_ERR_PLAN. Every entry's blob header is checked against the
 * entry (as w4a16_gemv checks it) at the start of the launch: if any does
 * not match, the launch writes no y at all and raises W4A16_CHAIN_ERR_BLOB.
 */
w4a16_status w4a16_gemv_chain(const void* plan, int32_t count, int32_t M, void* workspace,
                              size_t workspace_bytes, void* stream);

/*
 * w4a16_gemv_chain_timed - w4a16_gemv_chain, with the kernel's own start and
 * end times recorded into two caller-owned HIP events, as w4a16_gemv_timed.
 * Either event NULL -> W4A16_ERR_NULL; otherwise as w4a16_gemv_chain.
 */
w4a16_status w4a16_gemv_chain_timed(const void* plan, int32_t count, int32_t M, void* workspace,
                                    size_t workspace_bytes, void* stream, void* start_event, void* stop_event);

/*
 * w4a16_chain_status - host, blocking: the outcome of the chain calls enqueued
 * so far on `stream` with this workspace. Waits until the stream has drained,
 * reads the error word at W4A16_CHAIN_ERROR_OFFSET into *bits and, if `clear`
 * is nonzero and a bit was set, zero-fills the first
 * W4A16_CHAIN_WORKSPACE_BYTES of the workspace again (on `stream`, waited
 * for) so it can serve the next call.
 *   workspace, workspace_bytes, stream   as given to w4a16_gemv_chain
 * Returns W4A16_OK if the word is zero; W4A16_ERR_WAIT if
 * W4A16_CHAIN_ERR_WAIT is set; else W4A16_ERR_FORMAT (plan or blob header
 * mismatch). Host errors: NULL workspace or bits -> W4A16_ERR_NULL (bits
 * untouched); misaligned workspace -> W4A16_ERR_ALIGN; workspace_bytes too
 * small -> W4A16_ERR_SIZE; a failing wait or copy -> W4A16_ERR_HIP (*bits = 0).
 * Synchronises, so it is not for use under stream capture; the bits are
 * sticky across calls until cleared, so check after the last call of a
 * batch, or after every call when each result matters.
 */
w4a16_status w4a16_chain_status(const void* workspace, size_t workspace_bytes, void* stream, uint32_t* bits,
                                int32_t clear);

/*
 * w4a16_chain_launch_shape - host only: the three template arguments of the
 * kernel w4a16_gemv_chain launches for M, as profilers print its name
 * chain_kernel<out[0], out[1], out[2]>: activation rows, slots of the
 * workgroup's LDS ring of weight units, compute waves per workgroup.
 * Errors: NULL out -> W4A16_ERR_NULL; M outside 1..8 -> W4A16_ERR_SHAPE.
 */
w4a16_status w4a16_chain_launch_shape(int32_t M, int32_t out[3]);

/*
 * Weight-code variants: the same decode GEMV over other group codes.
 *
 * The Magnitude page (section 4.2, model conversion) compares the quantisation
 * types it measured: a symmetric 4-bit type (smallest, least accurate), the
 * 4-bit K-quant (the group-affine code above) and a 5-bit K-quant (more
 * accurate, about a quarter larger). The core-modules page puts edge weights
 * at INT8 or INT4 (section 5.1) and lists 4-bit and 8-bit weight
 * quantisation among the runtimes (section 5.2). No page defines these
 * formats; every codec below keeps groups of 32 consecutive k of one row
 * with binary16 parameters and no super-blocks. s and m are binary16
 * [N][K/32] arrays as in "Weight format"; G, T and S are as in "Packed
 * layout", S being the code region's size rounded up to 256 bytes.
 *
 * W4A16_CODEC_Q4 (0): the group-affine 4-bit code of w4a16_pack / w4a16_gemv.
 *
 * W4A16_CODEC_Q4_SYM (1): w_hat = s * (q - 8), q unsigned 4-bit.
 *   codes uint8 [N][K/2] as in "Weight format"; no min.
 *   packed: [0, N*K/2) the 4-bit code chunks of "Packed layout";
 *           [S, S + T*G*8) scale tiles: [T][G] entries of 8 bytes, row r of
 *           entry (t, g) in bytes 2r..2r+1 (rows at or beyond N are zero).
 *
 * W4A16_CODEC_Q5 (2): w_hat = s * q + m, q unsigned 5-bit (0..31).
 *   codes uint8 [N][K], one code per byte (a code above 31 is refused).
 *   packed: [0, N*K/2) the codes' low 4 bits as 4-bit code chunks;
 *           [S, S + T*G*16) fifth-bit tiles: [T][G] entries of 16 bytes, row
 *           r of entry (t, g) in the little-endian 32-bit word at bytes
 *           4r..4r+3, whose bit 4j + d (j = 0..7, d = 0..3) is bit 4 of the
 *           code of k = 32g + 8d + 2(j mod 4) + j/4;
 *           [S + T*G*16, S + 2*T*G*16) scale/min tiles as in "Packed layout".
 *
 * W4A16_CODEC_Q8_SYM (3): w_hat = s * q, q signed 8-bit (two's complement).
 *   codes int8 [N][K] (passed as their bytes); no min.
 *   packed: [0, N*K) codes: row n occupies K bytes, first the G 16-byte low
 *           halves of its groups (k = 32g .. 32g+15), then the G high halves
 *           (k = 32g+16 .. 32g+31); each byte is q + 128, and the
 *           little-endian 32-bit word e of a half holds k = 4e + i of that
 *           half with i = 0, 2, 1, 3 in bytes 0, 1, 2, 3;
 *           [S, S + T*G*8) scale tiles as for W4A16_CODEC_Q4_SYM.
 *
 * W4A16_CODEC_PAL4 (4): w_hat[n][k] = lut[n][q], q unsigned 4-bit: a palette
 *   of 16 binary16 values per output row (Core ML's palettisation, named in
 *   the core-modules page's runtime table, section 5.2, at per-row
 *   granularity: a table per group of 32 weights would outweigh them).
 *   codes uint8 [N][K/2] as in "Weight format"; the palettes binary16
 *   [N][16] are passed as `scale`; no min.
 *   packed: [0, N*K/2) codes: the canonical bytes, row after row (chunk
 *           (n, g) = the 16 bytes of group g, unchanged);
 *           [S, S + T*128) palette tiles: 128 bytes per tile t, entry c
 *           of row 4t + r at byte 8c + 2r (binary16, little-endian; rows at
 *           or beyond N are zero).
 */
typedef enum w4a16_codec {
  W4A16_CODEC_Q4 = 0,
  W4A16_CODEC_Q4_SYM = 1,
  W4A16_CODEC_Q5 = 2,
  W4A16_CODEC_Q8_SYM = 3,
  W4A16_CODEC_PAL4 = 4
} w4a16_codec;

/* Bytes of the packed blob of a codec (0 for an unknown codec or a bad N/K). */
size_t w4a16_codec_packed_bytes(int32_t codec, int32_t N, int32_t K);

/*
 * w4a16_codec_pack - host repacker of a codec (init time; touches no GPU).
 *   codes  host array in the codec's canonical layout (see above), read only
 *   scale  host binary16 bits [N][K/32], read only ([N][16] palettes for
 *          W4A16_CODEC_PAL4)
 *   min    host binary16 bits [N][K/32] for the affine codecs (0 and 2);
 *          ignored, and may be NULL, for the symmetric ones
 *   out    host buffer of at least w4a16_codec_packed_bytes(codec, N, K)
 *          bytes, owned by the caller, written completely
 * Errors: unknown codec or a 5-bit code above 31 -> W4A16_ERR_FORMAT (nothing
 * written); NULL -> W4A16_ERR_NULL; bad N/K -> W4A16_ERR_SHAPE; out_bytes too
 * small -> W4A16_ERR_SIZE. Codec 0 is exactly w4a16_pack.
 */
w4a16_status w4a16_codec_pack(int32_t codec, const uint8_t* codes, const uint16_t* scale, const uint16_t* min,
                              int32_t N, int32_t K, void* out, size_t out_bytes);

/*
 * w4a16_codec_gemv - y[M][N] = x[M][K] * w_hat^T for a blob written by
 * w4a16_codec_pack with the same codec, N and K. Arguments, ownership,
 * alignment (packed 256-byte aligned), overwrite semantics, determinism and
 * errors are those of w4a16_gemv, plus: unknown codec -> W4A16_ERR_FORMAT.
 * Codec 0 is exactly w4a16_gemv.
 */
w4a16_status w4a16_codec_gemv(int32_t codec, const void* x, const void* packed, float* y, int32_t M, int32_t N,
                              int32_t K, void* stream);

/* w4a16_codec_gemv with the kernel's own start and end recorded into two
 * caller-owned HIP events, as w4a16_gemv_timed. Either event NULL ->
 * W4A16_ERR_NULL. */
w4a16_status w4a16_codec_gemv_timed(int32_t codec, const void* x, const void* packed, float* y, int32_t M,
                                    int32_t N, int32_t K, void* stream, void* start_event, void* stop_event);

/*
 * w4a16_codec_launch_shape - host only: out[0] = groups of 32 k per lane,
 * out[1] = waves per workgroup, out[2] = passes over K of the kernel
 * w4a16_codec_gemv launches; for codecs 1..3 profilers name it
 * codec_kernel<codec, M, out[0], mode> with mode 0 (one wave per tile),
 * 1 (waves split K) or 2 (several passes over K). Codec 0: as
 * w4a16_launch_shape. Errors: NULL -> W4A16_ERR_NULL; unknown codec ->
 * W4A16_ERR_FORMAT; shape out of range -> W4A16_ERR_SHAPE.
 */
w4a16_status w4a16_codec_launch_shape(int32_t codec, int32_t M, int32_t N, int32_t K, int32_t out[3]);

/*
 * Decode attention over a quantised KV cache.
 *
 * The core-modules page (section 5.4, memory manager: KV budget) sizes the KV
 * cache of an 8B grouped-query model (32 layers, 8 KV heads, head size 128)
 * at 131,072 bytes per token in fp16, halved with INT8 and quartered with
 * INT4 values: at every decode step the whole cache is read once per layer,
 * the other bandwidth-bound operation of the step. The page defines no
 * format; the one here quantises per (token, KV head, group of 32 consecutive
 * dims) with binary16 parameters, like the weights:
 *   INT8 (bits = 8): v = s * q, q signed 8-bit;
 *   INT4 (bits = 4): v = s * q + m, q unsigned 4-bit.
 * One call computes one layer for one new token: for each query head h (KV
 * head g = h / (Hq / Hkv)),
 *   o[h][d] = sum_t softmax_t(q[h] . k_hat[t][g] / sqrt(128)) * v_hat[t][g][d].
 * The head size is 128; Hq / Hkv must be 1, 2, 4 or 8.
 *
 * Canonical cache arrays (host, per layer, tokens t < T):
 *   INT8: codes int8 [T][Hkv][128] (as bytes), scale binary16 [T][Hkv][4];
 *   INT4: codes uint8 [T][Hkv][64] (low nibble = even dim), scale and min
 *         binary16 [T][Hkv][4].
 * Packed cache (what w4a16_kv_pack writes): nb = ceil(T / 64) blocks of 64
 * tokens per KV head; records of R bytes ordered [g][block], R = 17,408
 * (INT8) or 10,240 (INT4). Inside the record of block b, slot i is token
 * 64b + i; slots at or beyond T are zero. Codes are packed in little-endian
 * 32-bit words: a word of four 8-bit elements holds element i in byte
 * (0, 2, 1, 3)[i], each as q + 128; a word of eight 4-bit elements holds
 * element i in byte (0, 2, 1, 3)[i % 4], in the low nibble for i < 4 and the
 * high nibble for i >= 4. (Masking such a word and the word shifted right by
 * 8 gives elements (0, 1) and (2, 3) as binary16 subnormal pairs.)
 *   INT8: [0, 8192) key codes: chunk c = dims 16c..16c+15 at 1024c, slot i's
 *         16 bytes at 1024c + 16i, word e = dims 16c + 4e .. + 3;
 *         [8192, 8704) key scales, 8 bytes per slot (groups 0..3);
 *         [8704, 9216) value scales, the same way;
 *         [9216, 17408) value codes: load 4h + u (h = 0, 1; u = 0..3) at
 *         9216 + 1024 (4h + u), lane l's 16 bytes at + 16l holding dim
 *         64h + l of slots 16u .. 16u + 15, word e = slots 16u + 4e .. + 3.
 *   INT4: [0, 4096) key codes: chunk c = group c (dims 32c..32c+31) at
 *         1024c, slot i's 16 bytes at + 16i, word w = dims 32c + 8w .. + 7;
 *         [4096, 5120) key (scale, min) pairs, 16 bytes per slot;
 *         [5120, 6144) value (scale, min) pairs, the same way;
 *         [6144, 10240) value codes: load 2h + u (h, u = 0, 1) at
 *         6144 + 1024 (2h + u), lane l's 16 bytes at + 16l holding dim
 *         64h + l of slots 32u .. 32u + 31, word w = slots 32u + 8w .. + 7.
 */

/* Bytes of one layer's packed cache (0 if bits is not 8 or 4, T < 1,
 * T > 2^24, or Hkv outside 1..4096). */
size_t w4a16_kv_packed_bytes(int32_t bits, int32_t T, int32_t Hkv);

/*
 * w4a16_kv_pack - host repacker of one layer's cache (touches no GPU).
 *   k_codes, v_codes  canonical codes (see above), read only
 *   k_scale, v_scale  binary16 bits [T][Hkv][4], read only
 *   k_min, v_min      binary16 bits [T][Hkv][4] for INT4; ignored (may be
 *                     NULL) for INT8
 *   out               host buffer of at least w4a16_kv_packed_bytes bytes,
 *                     owned by the caller, written completely
 * Errors: bits not 8 or 4 -> W4A16_ERR_FORMAT; NULL -> W4A16_ERR_NULL; bad
 * T/Hkv -> W4A16_ERR_SHAPE; out_bytes too small -> W4A16_ERR_SIZE.
 */
w4a16_status w4a16_kv_pack(int32_t bits, const uint8_t* k_codes, const uint16_t* k_scale, const uint16_t* k_min,
                           const uint8_t* v_codes, const uint16_t* v_scale, const uint16_t* v_min, int32_t T,
                           int32_t Hkv, void* out, size_t out_bytes);

/* Bytes of the device workspace w4a16_kv_attention needs for (T, Hq) (an
 * upper bound that holds on every device; 0 for a bad T or Hq). */
size_t w4a16_kv_workspace_bytes(int32_t T, int32_t Hq);

/*
 * w4a16_kv_attention - o[Hq][128] for one layer and one new token.
 *   q          device binary16 [Hq][128], 16-byte aligned (read only)
 *   kv         device copy of a w4a16_kv_pack blob for (bits, T, Hkv),
 *              256-byte aligned (read only)
 *   o          device fp32 [Hq][128], 16-byte aligned, overwritten
 *   workspace  device buffer of workspace_bytes >= w4a16_kv_workspace_bytes,
 *              16-byte aligned, owned by the caller; no initial contents
 *              needed; calls that share it must not run concurrently
 *   stream     hipStream_t to enqueue on
 * Two kernels are enqueued (the split attention pass and the merge of its
 * partials); the call never allocates or synchronises, and results are
 * bitwise repeatable. Errors (host side, before anything is enqueued): NULL
 * -> W4A16_ERR_NULL; bits, T or heads out of range -> W4A16_ERR_SHAPE;
 * misaligned pointer -> W4A16_ERR_ALIGN; workspace too small ->
 * W4A16_ERR_SIZE; o or the workspace intersecting an input or each other ->
 * W4A16_ERR_OVERLAP; launch rejected -> W4A16_ERR_HIP.
 */
w4a16_status w4a16_kv_attention(int32_t bits, const void* q, const void* kv, float* o, int32_t T, int32_t Hq,
                                int32_t Hkv, void* workspace, size_t workspace_bytes, void* stream);

/* w4a16_kv_attention with the start and end of its split attention kernel
 * (the dominant one; the merge kernel follows it) recorded into two
 * caller-owned HIP events. Either event NULL -> W4A16_ERR_NULL. */
w4a16_status w4a16_kv_attention_timed(int32_t bits, const void* q, const void* kv, float* o, int32_t T, int32_t Hq,
                                      int32_t Hkv, void* workspace, size_t workspace_bytes, void* stream,
                                      void* start_event, void* stop_event);

/* Bytes of the library's own partials array used by w4a16_kv_attention_static
 * (one per device, held until the process ends): room for
 * w4a16_kv_workspace_bytes(T, Hq) up to this size (8 MiB), e.g. T <= 129,024
 * tokens at Hq = 32 and T <= 64,512 at Hq = 64. */
#define W4A16_KV_STATIC_WORKSPACE_BYTES 8388608u

/*
 * w4a16_kv_attention_static - w4a16_kv_attention without a workspace
 * argument, for callers that cannot allocate device memory (code being
 * captured into a HIP graph, tight serving loops, harnesses that forbid
 * allocation). The partials go to an array the library holds in each
 * device's memory (W4A16_KV_STATIC_WORKSPACE_BYTES), whose device address is
 * looked up on the first call on a device. The call itself allocates
 * nothing. All calls on one device share that array and it keeps the last
 * call's partials: calls that can overlap on one device (other streams, other
 * threads) race and must be serialised by the caller (one stream, say).
 * Arguments, results (bitwise those of w4a16_kv_attention), ownership and
 * errors are those of w4a16_kv_attention, plus: w4a16_kv_workspace_bytes(T,
 * Hq) above W4A16_KV_STATIC_WORKSPACE_BYTES -> W4A16_ERR_SIZE (nothing
 * enqueued); the array's address not found -> W4A16_ERR_HIP.
 */
w4a16_status w4a16_kv_attention_static(int32_t bits, const void* q, const void* kv, float* o, int32_t T, int32_t Hq,
                                       int32_t Hkv, void* stream);

/* Host only: out[0] = query heads per KV head (the kernel's template argument,
 * kv_attn_kernel<bits, out[0]>), out[1] = blocks per workgroup, out[2] =
 * workgroups per KV head on the current device. NULL -> W4A16_ERR_NULL; bad
 * shape -> W4A16_ERR_SHAPE. */
w4a16_status w4a16_kv_launch_shape(int32_t bits, int32_t T, int32_t Hq, int32_t Hkv, int32_t out[3]);

/* Static, human-readable text for a status code (never NULL): the reason a
 * call was refused, as the contract table of the core-modules page (section
 * 5.7) asks of a runtime that turns away an input it does not cover. */
const char* w4a16_status_string(int32_t status);

#ifdef __cplusplus
}
#endif

#endif /* W4A16_H */
