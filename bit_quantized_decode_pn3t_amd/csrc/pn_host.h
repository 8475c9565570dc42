// pn_host.h - host-side helpers shared by the library's sources (argument
// checks, device facts, the kernel-variant census and the group plan).
// Internal to libpn.so; the public interface is include/pn.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/pn.h"

namespace pn {
namespace host {

// Kernel variants, as reported by pn_last_variant / pn_variant_name.
enum Variant {
    kVarNone = 0,
    kVarStream = 1,
    kVarGeneric = 2,
    kVarSmallMValu = 3,
    kVarDequant = 4,
    kVarGroupStream = 5,
    kVarSmallMMfma = 6,
    kVarGroupSmallMValu = 7,
    kVarGroupSmallMMfma = 8,
    kVarRows = 9,
    kVarGroupRows = 10,
    kVarRotate = 11,
    kVarPrefill = 12,
    kVarSmallMRows = 13,
    kVarGroupSmallMRows = 14,
    kVarBatchRows = 15,
    kVarBatchStream = 16,
    kVarPrefillGroup = 17,
};

extern thread_local int g_last_variant;

inline bool type_ok(int t) { return t == PN_PN3T || t == PN_PN4T; }
inline int wpb(int t) { return t == PN_PN3T ? 80 : 64; }
inline bool aligned4(const void *p) { return ((uintptr_t)p & 3) == 0; }

// Checks shared by every entry point that takes a packed matrix.
inline pn_status check_matrix(int t, const void *W, int64_t N, int64_t K)
{
    if (!type_ok(t) || !W) return PN_EINVAL;
    if (N < 1 || K < wpb(t) || K % wpb(t) != 0) return PN_ESHAPE;
    if ((uintptr_t)W & 1) return PN_EALIGN;
    if (N > INT32_MAX || K / wpb(t) * 34 > INT32_MAX) return PN_EUNSUPPORTED;
    return PN_OK;
}

// Devices the library keeps per-device facts for (ordinals 0..kMaxDevices-1;
// a call made with a higher ordinal current returns PN_EUNSUPPORTED).
constexpr int kMaxDevices = 64;

// Ordinal of the current device, or -1 if it cannot be used here.
int current_device();

// Compute units of the current device (256 if the query fails).  Filled once
// per device, thread-safe.
int device_cus();

// Run `set` (raising a kernel's LDS limit with hipFuncSetAttribute) once per
// device and flag; later calls return the first call's result.  Thread-safe.
enum AttrFlag { kAttrRows = 0, kAttrSmallM = 1, kAttrPrefill = 2, kAttrProbe = 3, kAttrCount = 4 };
bool once_per_device(AttrFlag f, bool (*set)());

// The calling thread's kernel selections (pn_set_gemv_kernel and
// pn_set_smallm_math act on the calling host thread only).
int gemv_kernel_choice();
int smallm_math_choice();

enum GroupKind { kGroupGemv = 0, kGroupSmallM = 1, kGroupGemvRows = 2 };

// pn_gemv_batch: the plan of a batch lives in one per-device buffer of
// kBatchBytes (a static device array): pool counters first (4 KiB apart),
// then the problem table, then the tile hand-out order of the row-tile kernel.
constexpr int kBatchMaxProblems = PN_BATCH_MAX_PROBLEMS;
constexpr int kBatchMaxTiles = PN_BATCH_MAX_ROWS / 16;  // 16-row tiles
constexpr size_t kBatchCounterBytes = 17 * 4096;
constexpr size_t kBatchTableOff = kBatchCounterBytes;
constexpr size_t kBatchTableBytes = 4096;
constexpr size_t kBatchLutOff = kBatchTableOff + kBatchTableBytes;
constexpr size_t kBatchBytes = kBatchLutOff + 4 * (size_t)kBatchMaxTiles;
static_assert(kBatchBytes == PN_BATCH_BYTES, "PN_BATCH_BYTES in pn.h");

}  // namespace host
}  // namespace pn

// A launch plan built by pn_group_create / pn_group_create_smallm.
struct pn_group {
    int kind;           // pn::host::GroupKind
    void *table;        // device copy of the per-problem records
    int count;
    int total_tiles;    // tiles (gemv_stream, gemm_stream) or waves (gemv_rows)
    int lds;            // dynamic LDS bytes of the launch
    int flags;          // kind-specific launch choice
    void *rot;          // problems with rotated inputs: RotJob list, then the rotated copies
    int rot_jobs;       // 1024-element blocks to rotate before the GEMV launch (0: none)
    int device;         // device current at creation: the plan's memory lives there
    int max_win;        // gemv_rows plans: most windows in one tile (bounds a wave's steps)
};

namespace pn {
namespace host {
// Launch a small-M group plan (pn_smallm.hip).
pn_status smallm_group_run(const pn_group *g, hipStream_t s);
// The row-tile M = 1 kernel (pn_gemv_rows.hip): whether it takes a problem,
// whether a launch of that many 16-row tiles is large enough for it, and
// its launches.
bool rows_ok(int t, const void *W, int64_t K, const void *x);
bool rows_pays(int64_t tiles);
int64_t rows_tiles(int64_t N);
pn_status rows_launch(int t, const void *W0, const void *W1, int64_t N, int64_t K, const void *x, float *y0,
                      float *y1, hipStream_t s);
pn_status rows_group_create(const pn_gemv_desc *descs, int count, pn_group **out);
pn_status rows_group_run(const pn_group *g, hipStream_t s);
// A batch (validated; every problem rows_ok, at most kBatchMaxTiles tiles) on
// the row-tile kernel, its plan written into `buf` (kBatchBytes, device) by a
// setup kernel ahead of the group launch, both on `s`.
pn_status rows_batch_launch(const pn_gemv_desc *descs, int count, uint8_t *buf, hipStream_t s);
// One block of a plan's activation rotation (pn_rotate.hip): src rotated
// into dst, PN_ROTATE_BLOCK fp16 elements each.
struct RotJob {
    const uint16_t *src;
    uint16_t *dst;
};
pn_status rotate_jobs_launch(const RotJob *jobs, int total, hipStream_t s);
}  // namespace host
}  // namespace pn
