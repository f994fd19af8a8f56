/*
 * moe_microbench.h -- measurement kernels of libmoe (no part of the layer).
 *
 * They give the figures that the layer's design rests on, from the same
 * library the layer runs in:
 *  - the rate at which a grid of blocks streams a contiguous buffer from HBM
 *    with 16-byte nontemporal loads (the read ceiling of the expert kernels,
 *    whose weights are read once per call);
 *  - the cost of a dependent kernel boundary (an empty kernel after another
 *    on one stream, or inside a HIP graph);
 *  - the cost of the grid-wide exchanges that one persistent kernel per layer
 *    (or per stack) would need in place of kernel boundaries: a count of
 *    arrivals, a grid barrier, and an all-to-all exchange of one word per block.
 * The pages run the layer as stream-ordered command buffers, one per step
 * ("48GB内存运行397B模型：Flash-Moe的极端量化与SSD流式加载实践", section "Metal
 * GPU管线：手写Kernel与FMA优化"; flash-moe README translation, "Pipeline mỗi lớp":
 * CMD1 .. CMD3 per layer); these kernels measure what that choice costs here.
 *
 * Conventions as in moe.h: device pointers owned by the caller, `stream` a
 * hipStream_t (NULL = default), arguments checked on the host before anything
 * is enqueued, negative moe_status_t values on error.
 */
#ifndef MOE_MICROBENCH_H
#define MOE_MICROBENCH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Read `bytes` (a multiple of 16, >= 16) of device memory at `src` (16-byte
 * aligned) once: the buffer is cut into `blocks` contiguous ranges (1 ..
 * 65536 blocks of 256 threads), each streamed by one block with
 * `in_flight` (1, 2, 4 or 8) 16-byte nontemporal loads per lane issued before
 * the first wait.  `sink` (device, 16 bytes) receives a value only if the
 * data XOR to a magic constant, so that the loads are not removed.
 */
int moe_mb_stream_read(const void *src, size_t bytes, int32_t blocks, int32_t in_flight, void *sink,
                       void *stream);

/*
 * As moe_mb_stream_read, with the dependency the layer's second and third
 * kernels have on the one before (the logits, then the selection): every lane
 * first loads 16 bytes of `dep` (2 KiB of device memory, 16-byte aligned,
 * typically the `out` of the previous call), and the block's loads start
 * off = (XOR of those words) & 4095 16-byte units into its range, so that no
 * load of the range issues before `dep` has arrived.  `src` must therefore
 * hold bytes + 64 KiB; a zero `dep` gives off = 0; a NULL `dep` means no
 * dependency (as the router's first loads have none).  At the end, block
 * b < 512 writes word b of `out` (2 KiB, 16-byte aligned): 0, unless its data
 * XOR to the sink's magic constant.  The rest as moe_mb_stream_read.
 */
int moe_mb_dependent_read(const void *src, size_t bytes, int32_t blocks, int32_t in_flight, const void *dep,
                          void *out, void *sink, void *stream);

/* An empty kernel of `blocks` (1 .. 65536) blocks of 256 threads. */
int moe_mb_empty(int32_t blocks, void *stream);

/*
 * Grid-wide exchange patterns of `blocks` blocks of 256 threads (1 .. 2048,
 * a multiple of `groups`); every block's wave 0 takes part.
 *   kind 0  arrivals: each block adds 1 to one of `groups` counters (block b
 *           uses counter b % groups), relaxed agent-scope atomics; no block
 *           waits.  The cost of finding the last block to arrive.
 *   kind 1  grid barrier: arrivals as in kind 0; the last arrival of each
 *           group adds 1 to a top counter, the last arrival there releases a
 *           generation word that every block polls.  Self-resetting.
 *   kind 2  as kind 1, the generation word written to `groups` lines and each
 *           block polling line b % groups (fewer pollers per address).
 *   kind 3  all-to-all: each block publishes one 64-bit word tagged with the
 *           call's generation; every block polls all of them until each
 *           carries that generation.  The generation advances when the last
 *           block leaves.
 *   kind 4  producers and consumers in one grid (blocks even, groups <= 64):
 *           the first blocks/2 blocks each publish a tagged word and then add
 *           1 to one of `groups` counters (release); each of the other blocks
 *           polls the counters until every producer has arrived, then reads
 *           and checks every producer's word (a router's logits reaching the
 *           expert blocks of the same launch).  Producers never wait, so the
 *           grid need not be resident all at once.
 * Polls are relaxed agent-scope loads.  The barriers (kinds 1, 2) release
 * and acquire (one acquire fence once the wait succeeds); the exchanges of
 * tagged words (kinds 3, 4) are relaxed throughout, as their words validate
 * themselves.
 * `buf`: device memory of at least moe_mb_exchange_bytes(blocks, groups)
 * bytes, 256-byte aligned, zeroed once before the first call (for example by
 * hipMemset); every call leaves it valid for the next.  Calls on one `buf`
 * must be stream-ordered.  Every wait is bounded (about 2^18 polls); a wait
 * that gives up raises a flag in the first word of `buf` (read it with
 * moe_mb_exchange_failures after synchronising) and the kernel ends normally.
 * The blocks must be resident together for kinds 1-3 to complete without
 * giving up: at most 2 blocks per compute unit.  A word that kind 4 finds
 * without its tag also counts as a give-up.
 */
int moe_mb_exchange(int32_t kind, int32_t blocks, int32_t groups, void *buf, size_t buf_bytes, void *stream);

/* Bytes of `buf` that moe_mb_exchange needs (0 for invalid arguments). */
size_t moe_mb_exchange_bytes(int32_t blocks, int32_t groups);

/* Number of bounded waits that gave up since `buf` was zeroed (reads device
 * memory with a blocking copy; call after the work has completed). */
int moe_mb_exchange_failures(const void *buf, uint32_t *failures);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MICROBENCH_H */
