/*
 * gbsa_slot_trace.h -- readout of libgbsa_slot_trace.so, a diagnostic build of libgbsa (the
 * same entry points, built with GBSA_SLOT_TRACE defined) whose 256-row DMA prefill kernel
 * (more than 256 packed rows per unit, 16-bit key/value) time-stamps its items.
 *
 * In each forward launch, the first workgroup to meet a unit of at least 12 visible pages
 * records, for each of its 8 waves, the shader clock (s_memtime, the clock the waves run at)
 * at every item boundary of that unit's loop: 1 softmax item start, 2 softmax item end,
 * 3 before the barrier that follows it, 4 after that barrier, 5 MFMA item start, 6 MFMA item
 * end (its loads waited for), 7 after the barrier that follows it. The kernel is the
 * FlashAttention article's (ai6s.net) "three steps" loop over the selected blocks, two wave
 * groups alternating its matrix and softmax halves; the stamps show how long each half takes
 * and how long each group waits for the other.
 *
 * Record layout: 8 waves x 1024 words of uint64, wave-major; word = (code << 56) | (clock &
 * (2^56 - 1)), events in order, unused words 0. Stamps of different workgroups are not
 * comparable (each XCD has its own counter); within one workgroup they are.
 *
 * Both calls act on the current device and return 0 or a hipError_t code; they synchronise
 * with the device (plain symbol copies), so call them outside timed regions.
 */
#ifndef GBSA_SLOT_TRACE_H_
#define GBSA_SLOT_TRACE_H_

#ifdef __cplusplus
extern "C" {
#endif

/* Copy the record (8 * 1024 uint64, 64 KiB) to host memory `host_dst`. */
int gbsa_slot_trace_read(unsigned long long* host_dst);

/* Clear the record and the claim, so that the next launch records again. */
int gbsa_slot_trace_reset(void);

#ifdef __cplusplus
}
#endif

#endif /* GBSA_SLOT_TRACE_H_ */
