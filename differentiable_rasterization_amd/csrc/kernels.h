// Host-side launchers shared between translation units of libgsmi (not part of the ABI).
#pragma once

#include "common.h"

namespace gsi {

gs_status check_gaussians(const gs_gaussians *g);

// Backward through projection and colour evaluation (defined in project.hip).
gs_status launch_project_bwd(const gs_gaussians *g, const gs_camera *cam, const gs_raster_params *p,
                             const float *grads2d, gs_param_grads *out, hipStream_t stream);

// Device-wide exclusive scan of m uint32 values (in place allowed).  If total != NULL
// the 64-bit sum is written there.  partials: scan_partials_len(m) uint32.
int64_t scan_partials_len(int64_t m);
gs_status exclusive_scan_u32(const uint32_t *in, uint32_t *out, int64_t m, uint32_t *partials,
                             unsigned long long *total, hipStream_t stream);

// Exclusive scan of m >= 1 uint32 values (in place allowed) in one launch, by look-back
// over the published sums of earlier tiles.  status [lb_scan_tiles(m)] uint64 and *ticket
// must be zero on entry (each scan needs its own).  If total != NULL the 64-bit sum is
// written there.  With clear != NULL the scan also sets clear[x] = 0 for every x below
// min(sum, clear_lim) (each tile zeroes its own output range, coalesced).
int64_t lb_scan_tiles(int64_t m);
gs_status lb_scan_u32(const uint32_t *in, uint32_t *out, int64_t m, unsigned long long *status, uint32_t *ticket,
                      unsigned long long *total, hipStream_t stream, uint32_t *clear = nullptr,
                      int64_t clear_lim = 0);
// The same over the high 32 bits of m uint64 values (in: 16-byte aligned).  With sel !=
// NULL, the input is in_alt instead of in when *sel != 0 (read on the device).
gs_status lb_scan_hi32(const uint64_t *in, uint32_t *out, int64_t m, unsigned long long *status, uint32_t *ticket,
                       unsigned long long *total, hipStream_t stream, const uint64_t *in_alt = nullptr,
                       const uint32_t *sel = nullptr);

// Stable LSD radix sort of (key, value) uint32 pairs on the low `bits` bits of the key,
// 8 bits per pass, ping-ponging between (ka, va) and (kb, vb).  Returns in *in_b whether
// the sorted result ended in (kb, vb).  hist: radix_hist_len(m) uint32; scan_status
// [radix_scan_status_len(m, bits)] uint64 and scan_tickets [passes] must be zero on entry.
// If m_dev is given, the number of elements is min(m, *m_dev), read on the device (m
// sizes the launches).
int64_t radix_hist_len(int64_t m);
int64_t radix_scan_status_len(int64_t m, int bits);
gs_status radix_sort_u32(uint32_t *ka, uint32_t *va, uint32_t *kb, uint32_t *vb, int64_t m, int bits,
                         uint32_t *hist, unsigned long long *scan_status, uint32_t *scan_tickets, bool *in_b,
                         hipStream_t stream, const unsigned long long *m_dev = nullptr);
// The same with 64-bit values.  xf (device, may be NULL; 32-bit sorts only): kRadixXfWords
// words, zero before the call.  With xf, the sort finds the range of the keys other than 0xFFFFFFFF
// on the device; when they lie within about 2^24 of each other (the exact test is in
// sort.hip), it takes three passes instead of four and the result ends in (kb, vb): then
// xf[1] != 0 after the sort (read it on the device; *in_b reports the four-pass case).
// low_out (device, may be NULL; not with xf): the last pass also writes the low 32 bits of
// each sorted value there; nothing is written when m <= 1 (no pass runs).
constexpr int kRadixXfWords = 32 * 33;
gs_status radix_sort_u32_u64(uint32_t *ka, uint64_t *va, uint32_t *kb, uint64_t *vb, int64_t m, int bits,
                             uint32_t *hist, unsigned long long *scan_status, uint32_t *scan_tickets, bool *in_b,
                             hipStream_t stream, const unsigned long long *m_dev = nullptr,
                             uint32_t *xf = nullptr, uint32_t *low_out = nullptr);

// Fills n int32 values with `value` (a kernel, not a memset, so it may be captured in graphs).
gs_status fill_i32(int32_t *p, int64_t n, int32_t value, hipStream_t stream);
gs_status fill_f32(float *p, int64_t n, float value, hipStream_t stream);

}  // namespace gsi
