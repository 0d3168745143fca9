/*
 * oracle.c -- the CPU oracle for the batched descriptor copy.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file.  It may be used only by tests/, by the smoke check in
 * __graft_entry__.py and by the cpu_baseline leg of bench.py.  It shares no
 * code, header or helper with block_copy_amd/csrc/.
 *
 * What it computes.  A batch is a list of n descriptors (src_addr, dst_addr,
 * size): raw device-visible addresses and a byte count.  The method moves
 * every descriptor's bytes from src to dst; the result it reaches is exactly
 * that of one memcpy per descriptor, applied in list order:
 *   - vLLM PR #42212 report ("[Perf] Triton fast path for small CPU->GPU
 *     swap_blocks_batch in the offloading connector"), section "key source
 *     snippet": each job stores word idx of dst equal to word idx of src for
 *     every idx below size/8, and the unit test of that PR checks that the
 *     copied bytes equal the source bytes;
 *   - FreeToken issue #751 ("gather missed experts with a few TMA bulk-copy
 *     CTAs"), sections "What we changed" and "Correctness evidence": the new
 *     gather moves the same bytes as the upstream kernel and is byte-exact;
 *   - PegaFlow issue #408 ("Kernel transfer backend causes decode TPOT tail
 *     spikes under concurrent KV transfers"), section "Relevant
 *     implementation": the kernel backend and the per-range memcpy backend
 *     are interchangeable transports for the same blocks.
 *
 * Because the caller's addresses point into GPU or mapped host memory, the
 * oracle works on host *images*: each arena the batch touches is given as
 * (base address, length, host byte image).  An address is translated to an
 * image pointer by finding the arena that holds [addr, addr+size).  The copy
 * itself is then a plain memcpy per descriptor, in list order, on the
 * uncoalesced input.  Nothing is chunked, merged, reordered or threaded.
 *
 * Inputs that the contract leaves undefined (overlapping destinations, a
 * destination that overlaps a source) are not given to the oracle.
 */
#include <stdint.h>
#include <string.h>

typedef struct {
    uint64_t base; /* device-visible address of the arena's first byte */
    uint64_t len;  /* bytes */
    uint8_t *img;  /* host image of the arena */
} oracle_arena_t;

/* Image pointer for [addr, addr+size) or NULL if no single arena holds it. */
static uint8_t *oracle_locate(const oracle_arena_t *arenas, int n_arenas,
                              uint64_t addr, uint64_t size)
{
    for (int a = 0; a < n_arenas; ++a) {
        const oracle_arena_t *r = &arenas[a];
        if (addr >= r->base && size <= r->len && addr - r->base <= r->len - size)
            return r->img + (addr - r->base);
    }
    return NULL;
}

/*
 * oracle_copy: for i = 0 .. n-1, memcpy(dst_image(dst[i]), src_image(src[i]), size[i]).
 *
 * Returns 0, or -(i+1) if descriptor i names an address outside every arena
 * (a harness bug; nothing from descriptor i on is applied).  *bytes_moved
 * receives the sum of the sizes applied.
 */
int64_t oracle_copy(const uint64_t *src, const uint64_t *dst, const uint64_t *size,
                uint64_t n,
                const oracle_arena_t *src_arenas, int n_src,
                const oracle_arena_t *dst_arenas, int n_dst,
                uint64_t *bytes_moved)
{
    uint64_t moved = 0;
    for (uint64_t i = 0; i < n; ++i) {
        if (size[i] == 0)
            continue;
        const uint8_t *s = oracle_locate(src_arenas, n_src, src[i], size[i]);
        uint8_t *d = oracle_locate(dst_arenas, n_dst, dst[i], size[i]);
        if (s == NULL || d == NULL) {
            if (bytes_moved)
                *bytes_moved = moved;
            return -(int64_t)(i + 1);
        }
        memcpy(d, s, size[i]);
        moved += size[i];
    }
    if (bytes_moved)
        *bytes_moved = moved;
    return 0;
}
