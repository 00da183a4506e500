/*
 * lutgemm.h -- C ABI of the MI355X (gfx950) BCQ LUT-GEMV library.
 *
 * The operation (LUT-GEMM, Park et al.; Elamur card "LUT-GEMM -- paper by
 * Park et al. (2022)", section "Summary"; pith.science page of the same title,
 * original abstract): y = W_hat * x for fp16 activations x and a weight matrix
 * held in binary-coding quantization (BCQ),
 *
 *     W_hat[j][k] = sum_{i<q} alpha[i][j][k/g] * b_i[j][k]  (+ offset[j][k/g]),
 *     b_i[j][k] in {-1, +1},
 *
 * computed without ever forming W_hat: for every 8-input chunk of x all 256
 * signed sums are built once into a table, and each weight byte (the 8 sign
 * bits of one plane, row and chunk) selects its sum, which is scaled by alpha
 * and accumulated (card section "Interesting ideas: Lookup tables instead of
 * multiplications"). Scales are group-wise with group size g (card section
 * "Interesting ideas: Group size as a separate hyper-parameter"); the optional
 * per-group offset lets a uniform int-q matrix be held exactly as BCQ (card
 * section "Interesting ideas: One format for many schemes").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Plain pointers and sizes only; no C++ or framework types cross this ABI,
 *   and no C++ exception escapes it. Every function returns a status code
 *   (lutgemm_status) unless stated otherwise.
 * - The caller owns every buffer, host and device. The library never
 *   allocates, frees or synchronizes device memory or streams.
 * - fp16 values are passed as their IEEE binary16 bit patterns (uint16_t).
 * - Logical (unpacked) weight format, used as packer input:
 *     bits   uint8  [q][N][K/8]  bit t (least significant first) of byte c of
 *                                row j in plane i is the sign of weight
 *                                (j, 8c+t): 1 means +1, 0 means -1;
 *     alpha  fp16   [q][N][K/g]
 *     offset fp16   [N][K/g]     (only when has_offset)
 * - Packed (device) format, produced by bcq_pack / bcq_pack_uniform and read
 *   by lutgemm_run. Rows are padded to Npad = 16*ceil(N/16) and 8-input
 *   chunks to 64*ceil(K/512); padding bytes and scales are zero.
 *     bits   byte   [ceil(K/512)][Npad/16][q][1024]  one block per (input
 *                                tile, row tile, plane): 64 lane blocks of 16 bytes;
 *                                lane block 16*r4 + c4 holds rows 4*r4 + a and
 *                                chunks 4*c4 + b (a, b < 4) at byte 4*a + b
 *     alpha  fp16   [Npad/16][K/g][q][16]
 *     offset fp16   [Npad/16][K/g][16]
 * - Shape rules (else LUTGEMM_ERR_SHAPE): N >= 0, K >= 0, K % 8 == 0,
 *   1 <= q <= 8, g >= 8, g % 8 == 0, K % g == 0 (when K > 0),
 *   has_offset in {0, 1}, N and K below 2^30, 0 <= m <= 65535. For
 *   lutgemm_run and lutgemm_workspace_size, each of the packed bits, packed
 *   alpha, packed offset and x (m*K fp16) must also be smaller than 4 GiB.
 */
#ifndef LUTGEMM_H
#define LUTGEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LUTGEMM_ABI_VERSION 1

typedef enum lutgemm_status {
  LUTGEMM_OK = 0,
  LUTGEMM_ERR_NULL = 1,        /* a required pointer is NULL                         */
  LUTGEMM_ERR_SHAPE = 2,       /* N, K, q, g, has_offset or m breaks the shape rules */
  LUTGEMM_ERR_VALUE = 3,       /* code/zero-point >= 2^q, non-finite scale, alpha or */
                               /* offset, or a rewritten scale that overflows fp16   */
  LUTGEMM_ERR_BUFFER = 4,      /* an output buffer or the workspace is too small     */
  LUTGEMM_ERR_ALIGN = 5,       /* a device pointer is not aligned as required        */
  LUTGEMM_ERR_UNSUPPORTED = 6, /* the current device is not gfx950 (the environment  */
                               /* variable LUTGEMM_FAKE_ARCH, a debugging aid,      */
                               /* replaces the name the device reports), or the     */
                               /* call needs a feature this build lacks             */
  LUTGEMM_ERR_HIP = 7,         /* a HIP runtime call or a kernel launch failed       */
  LUTGEMM_ERR_INTERNAL = 8     /* unexpected internal failure                        */
} lutgemm_status;

typedef struct lutgemm_shape {
  int32_t N;          /* output rows                                 */
  int32_t K;          /* inputs per row (reduction length)           */
  int32_t q;          /* sign planes, 1..8                           */
  int32_t g;          /* inputs per scale group                      */
  int32_t has_offset; /* 1 if a per-(row, group) offset is present   */
} lutgemm_shape;

/* LUTGEMM_ABI_VERSION of the built library. Never fails. */
int lutgemm_abi_version(void);

/* Static, NUL-terminated description of a status code. Never NULL. */
const char* lutgemm_status_string(int status);

/* Validate a shape against the shape rules. */
int lutgemm_check_shape(const lutgemm_shape* s);

/* Sizes of the packed format for shape *s: bytes of packed bits, and counts
 * (fp16 elements) of packed alpha and packed offset (0 without offset).
 * Any output pointer may be NULL. Host only; no HIP call. */
int lutgemm_packed_sizes(const lutgemm_shape* s, size_t* bits_bytes,
                         size_t* alpha_count, size_t* offset_count);

/* Device workspace lutgemm_run needs for shape *s at batch m, in bytes (0 when
 * none). It is needed when the input dimension is split across workgroups:
 * it holds arrival counters (at its start) and fp32 partial sums. It must be
 * zero-filled before its first use (lutgemm_workspace_init); every call that
 * completes leaves the counters zero again, so one workspace then serves any
 * later call whose requirement it meets. Host only; no HIP call. */
int lutgemm_workspace_size(const lutgemm_shape* s, int32_t m, size_t* bytes);

/* Zero-fill `bytes` of device workspace on `stream` (a hipStream_t; NULL for the
 * default stream), asynchronously, with a kernel (no memset node, so it can be
 * captured in a graph). */
int lutgemm_workspace_init(void* d_workspace, size_t bytes, void* stream);

/* Pack a BCQ matrix from the logical format into the device format. The
 * logical format is the method's weight representation: q sign planes with
 * one scale per (plane, row, group of g inputs) and an optional per-group
 * offset (Elamur card "LUT-GEMM -- paper by Park et al. (2022)", sections
 * "Summary" and "Interesting ideas: Group size as a separate
 * hyper-parameter"; pith.science page of the same title, original abstract).
 * The packed layout is this library's own (see the conventions above).
 * Host only (CPU), deterministic: the output bytes are fully determined by
 * the inputs. `offset` must be non-NULL exactly when s->has_offset.
 * Rejects non-finite alpha/offset values (LUTGEMM_ERR_VALUE) and output
 * buffers smaller than lutgemm_packed_sizes (LUTGEMM_ERR_BUFFER). On error
 * nothing has been written. */
int bcq_pack(const lutgemm_shape* s, const uint8_t* bits, const uint16_t* alpha,
             const uint16_t* offset, uint8_t* out_bits, size_t out_bits_bytes,
             uint16_t* out_alpha, size_t out_alpha_count, uint16_t* out_offset,
             size_t out_offset_count);

/* Rewrite a uniform int-q matrix, W[j][k] = scale[j][k/g] * (codes[j][k] -
 * zero[j][k/g]), as BCQ with q planes plus offset, and pack it (card sections
 * "Summary" and "Interesting ideas: One format for many schemes").
 *   codes uint8 [N][K] (< 2^q), scale fp16 [N][K/g], zero uint8 [N][K/g] (< 2^q).
 * Plane i holds bit i of the code, alpha_i = scale * 2^(i-1) and
 * offset = scale * ((2^q - 1)/2 - zero), each rounded to the nearest fp16
 * (ties to even). s->has_offset must be 1. *n_rounded (may be NULL) receives
 * the number of groups for which any of these values was not exactly
 * representable in fp16. Host only; on error nothing has been written. */
int bcq_pack_uniform(const lutgemm_shape* s, const uint8_t* codes,
                     const uint16_t* scale, const uint8_t* zero,
                     uint8_t* out_bits, size_t out_bits_bytes,
                     uint16_t* out_alpha, size_t out_alpha_count,
                     uint16_t* out_offset, size_t out_offset_count,
                     size_t* n_rounded);

/* y = W_hat x on the current HIP device, enqueued on `stream` (a hipStream_t;
 * NULL for the default stream). Asynchronous: returns after the launch.
 * This is the LUT-GEMM product (Elamur card "LUT-GEMM -- paper by Park et al.
 * (2022)", sections "Summary" and "Interesting ideas: Lookup tables instead
 * of multiplications"; pith.science page of the same title, original
 * abstract): fp16 activations times the BCQ weights, with the 256 signed sums
 * of every 8-input chunk of x computed once per table and selected by each
 * weight byte, so the weights are never expanded.
 *   d_bits, d_alpha, d_offset: packed device format (d_offset only when
 *       s->has_offset, else ignored);
 *   d_x  fp16 [m][K] row-major;  d_y  fp16 [m][N] row-major, overwritten;
 *   d_workspace: at least lutgemm_workspace_size bytes, zero-filled before its
 *       first use (may be NULL when that size is 0); calls that overlap in time
 *       must not share a workspace. The size query assumes a full 256-CU
 *       MI355X; on a device with another number of compute units the launch
 *       chooses its own work split and limits it to workspace_bytes.
 * Alignment (else LUTGEMM_ERR_ALIGN): d_bits, d_x and d_workspace 16 bytes,
 * d_alpha and d_offset 4 bytes, d_y 2 bytes.
 * Arithmetic: table entries, scaling and accumulation in fp32; y rounded to
 * fp16 to nearest-even. The launch configuration (waves, rows per item, batch
 * rows per item, split of the input dimension) is chosen from the shape and m;
 * results are bitwise reproducible for a fixed shape and batch. (The
 * environment variable LUTGEMM_TILE, a tuning aid, overrides that choice; the
 * results then stay within the same tolerance but may round differently.)
 * All argument checks run before any HIP call; on error nothing is launched.
 * Faults inside the kernel surface at the caller's next synchronization of
 * `stream`. */
int lutgemm_run(const lutgemm_shape* s, int32_t m, const void* d_bits,
                const void* d_alpha, const void* d_offset, const void* d_x,
                void* d_y, void* d_workspace, size_t workspace_bytes,
                void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * product as lutgemm_run, with the same operands, alignment rules, status codes
 * and asynchrony, but no workspace argument and no allocation of any kind.
 * Where the input dimension is split across workgroups, the arrival counters
 * and fp32 partial sums live in a fixed scratch array inside the library, one
 * per GPU, held until the process ends; its size is
 * lutgemm_noalloc_scratch_bytes() (4 MiB). The launch is chosen among those
 * whose partial sums fit that scratch (a smaller split, down to none, when the
 * best one would not), so every valid shape runs; a split forced through the
 * LUTGEMM_TILE tuning override that would not fit is refused with
 * LUTGEMM_ERR_BUFFER before any HIP call. The first call on a device clears
 * the scratch's counters with a kernel on `stream`; every completed call leaves
 * them zero. All calls on one GPU share its scratch, so calls that overlap in
 * time on one GPU (on different streams, or from different threads) race and
 * must be ordered by the caller. Results can differ in rounding from
 * lutgemm_run's when the two choose different splits, and stay within the
 * same tolerance. */
int lutgemm_run_noalloc(const lutgemm_shape* s, int32_t m, const void* d_bits,
                        const void* d_alpha, const void* d_offset, const void* d_x,
                        void* d_y, void* stream);

/* Size in bytes of the scratch array lutgemm_run_noalloc uses on each GPU.
 * Never fails; host only. */
size_t lutgemm_noalloc_scratch_bytes(void);

/* The launch chosen for shape *s and batch m on a device with `cus` compute
 * units, its split limited to `workspace_bytes` of workspace, after the
 * LUTGEMM_TILE override if set. lutgemm_run's launch is the plan for
 * (256, SIZE_MAX) on a full 256-CU MI355X and for (the device's count, the
 * workspace passed) on any other; lutgemm_run_noalloc's is the plan for (the
 * device's count, lutgemm_noalloc_scratch_bytes()). For tracing and tuning;
 * host only, no HIP call.
 * Table kinds (the card's section "Interesting ideas: Lookup tables instead of
 * multiplications" defines the 256-entry table of an 8-input chunk):
 *   LUTGEMM_TABLES_SINGLE  one table per batch row, two buffers;
 *   LUTGEMM_TABLES_PAIRED  the tables of two batch rows interleaved entry by
 *                          entry, one buffer;
 *   LUTGEMM_TABLES_HALF    as paired, holding only the 128 entries with bit 7
 *                          clear (entry b ^ 0xFF is minus entry b), two buffers;
 *   LUTGEMM_TABLES_NIBBLE  16-entry tables of 4-input halves of each chunk,
 *                          a byte's entry being the sum of its two halves';
 *   LUTGEMM_TABLES_SPLIT   paired tables built for half an input tile at a
 *                          time (32 chunks), two buffers;
 *   LUTGEMM_TABLES_PAIRED_MFMA  paired tables whose entries are computed by
 *                          matrix-core instructions (the 256 x 8 sign matrix
 *                          times the tile's activations);
 *   LUTGEMM_TABLES_SIGN_MFMA  no tables: each sign plane times up to 32 batch
 *                          rows of x on the matrix cores, the same signed sums
 *                          per scale group (batches of several rows).
 * Fields of a plan with no launch (m == 0, N == 0 or K == 0) are zero.
 * Errors: NULL when s or out is NULL, SHAPE as for lutgemm_run or when
 * cus < 1, INTERNAL when no kernel instance fits. */
enum {
  LUTGEMM_TABLES_SINGLE = 0,
  LUTGEMM_TABLES_PAIRED = 1,
  LUTGEMM_TABLES_HALF = 2,
  LUTGEMM_TABLES_NIBBLE = 3,
  LUTGEMM_TABLES_SPLIT = 4,
  LUTGEMM_TABLES_PAIRED_MFMA = 5,
  LUTGEMM_TABLES_SIGN_MFMA = 6
};
typedef struct lutgemm_plan {
  int32_t tables;         /* LUTGEMM_TABLES_*                                   */
  int32_t waves;          /* wave64s per workgroup                              */
  int32_t rows_per_wave;  /* row tiles (16 rows) a wave looks up per step       */
  int32_t batch_rows;     /* batch rows per work item                           */
  int32_t row_tiles;      /* row tiles per work item                            */
  int32_t split;          /* workgroups sharing one row block's input dimension */
  int32_t x_in_lds;       /* 1: the whole of x is staged in LDS once            */
  int32_t reserved;
  int64_t items;          /* work items (row block, batch group, split)         */
  int64_t workgroups;     /* workgroups launched                                */
  uint64_t workspace_bytes;
} lutgemm_plan;
int lutgemm_query_plan(const lutgemm_shape* s, int32_t m, int32_t cus, size_t workspace_bytes,
                       lutgemm_plan* out);

/* Phase timestamps, a tracing aid. In the library built with phase tracing
 * (liblutgemm_trace.so, built beside liblutgemm.so from the same sources),
 * every launch of the GEMV kernels that starts after this call writes, for
 * each workgroup w below bytes / 64, stamps of the GPU's constant 100 MHz clock
 * into the device buffer d_buffer as uint64 [w][8]: index 0 at the
 * workgroup's start, 1 when x is staged in LDS (batch 1), 2 when the first
 * table is built, 3 when the first step is done, 4 when its last lookups are
 * done, 5 at its end; a launch leaves the indices it does not pass as they
 * were. Results are those of the regular library. NULL detaches. The buffer
 * belongs to the caller and must stay valid while traced launches run;
 * launches that overlap in time write the same buffer.
 * Errors: ALIGN when d_buffer is not 8-byte aligned; the regular library
 * returns UNSUPPORTED and records nothing. Host only (no HIP call). */
int lutgemm_trace_attach(void* d_buffer, size_t bytes);

/* Storage in bits of the matrix of shape *s: q sign bits per weight, one fp16
 * scale per (plane, row, group of g) and one fp16 offset per (row, group) when
 * s->has_offset (Elamur card, section "Interesting ideas: Group size as a
 * separate hyper-parameter": scales count toward the storage). Host only. */
int bcq_footprint_bits(const lutgemm_shape* s, uint64_t* bits);

/* Group sizes for a storage target (same card section: q and g are chosen
 * together for a target compression). For each plane count q = 1..8, the
 * smallest g (a divisor of K, multiple of 8: the finest scales) whose footprint
 * for an N x K matrix is at most max_bits_per_weight * N * K bits:
 * out_g[q-1] = g and out_bits[q-1] = the footprint, or both 0 when no g fits.
 * out_g and out_bits hold 8 entries each. Errors: LUTGEMM_ERR_NULL,
 * LUTGEMM_ERR_SHAPE (N < 1, K < 8, K % 8, N or K >= 2^30, has_offset not 0/1),
 * LUTGEMM_ERR_VALUE (target not in (0, 1e6]). Host only. */
int bcq_search_group_sizes(int64_t N, int64_t K, int32_t has_offset, double max_bits_per_weight,
                           int32_t* out_g, uint64_t* out_bits);

/* Binary-coding quantization of an fp16 matrix into the logical BCQ format
 * that bcq_pack takes (the format of the card's sections "Summary" and
 * "Interesting ideas: Group size as a separate hyper-parameter"; the pages name
 * the quantizer only by reference, so the method is this library's reading):
 * greedy per (row, group): plane by plane, alpha_i = the mean absolute residual
 * rounded to fp16, b_i = its sign (0 counts as +1); then `iters` rounds of
 * alternating refinement (least-squares refit of the q scales, rounded to fp16,
 * kept unchanged when the system is singular or a scale overflows fp16; then each weight
 * takes its nearest sign combination, lowest index on ties).
 *   w     fp16 [N][K] (finite)      bits  uint8 [q][N][K/8]  (as for bcq_pack)
 *   alpha fp16 [q][N][K/g]          *sq_error (may be NULL) = sum (w - W_hat)^2
 * s->has_offset must be 0; 0 <= iters <= 1000. Errors: LUTGEMM_ERR_SHAPE,
 * LUTGEMM_ERR_NULL, LUTGEMM_ERR_BUFFER (outputs too small), LUTGEMM_ERR_VALUE
 * (non-finite w or iters out of range); on error nothing has been written.
 * Deterministic; host only (CPU threads). */
int bcq_quantize(const lutgemm_shape* s, const uint16_t* w, int32_t iters, uint8_t* bits,
                 size_t bits_bytes, uint16_t* alpha, size_t alpha_count, double* sq_error);

/* The comparison point, not the method: y = W_hat x by expanding every weight
 * to fp16 (W_hat[j][k] = sum_i +-alpha[i][j][k/g] (+ offset), packed fp16 adds)
 * and taking fp16 dot products with fp32 accumulation, the way dequantizing
 * weight-only kernels work (Elamur card "LUT-GEMM -- paper by Park et al.
 * (2022)", section "Summary": LUT-GEMM is set against kernels that expand
 * low-bit weights to FP16 before multiplying). Same arguments, packed format,
 * alignment rules and status codes as lutgemm_run, without a workspace; y is
 * within the same tolerance of the exact product (the weight sums are rounded
 * to fp16). Asynchronous on `stream`; all argument checks run before any HIP
 * call. */
int bcq_dequant_gemv(const lutgemm_shape* s, int32_t m, const void* d_bits,
                     const void* d_alpha, const void* d_offset, const void* d_x,
                     void* d_y, void* stream);

/* Measurement aid, not part of the method: read `bytes` of device memory at
 * d_src once with 128-bit loads (one workgroup of 16 waves per compute unit,
 * all workgroups reading one window of memory together, four loads in flight
 * per thread), non-temporal when `nontemporal` is 1. This is the achievable
 * HBM read rate the GEMV's bandwidth is compared against. The loaded values are
 * folded and, almost never, written to d_sink (uint32, at least one entry per
 * compute unit, sink_count entries). Alignment: d_src 16 bytes, d_sink 4.
 * bytes < 4 GiB - 64 KiB (else LUTGEMM_ERR_SHAPE); reads past `bytes` inside
 * the last 64 KiB block return zero without touching memory. Asynchronous on
 * `stream`. Errors: LUTGEMM_ERR_NULL, LUTGEMM_ERR_ALIGN, LUTGEMM_ERR_VALUE
 * (nontemporal not 0/1), LUTGEMM_ERR_BUFFER (sink_count too small),
 * LUTGEMM_ERR_HIP. */
int lutgemm_stream_read(const void* d_src, size_t bytes, uint32_t* d_sink, size_t sink_count,
                        int nontemporal, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LUTGEMM_H */
