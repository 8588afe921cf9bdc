/* Internal helpers shared by the library's translation units (not installed). */
#ifndef PKV_INTERNAL_H
#define PKV_INTERNAL_H

#include "pagedkv.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Record a printf-style message as this thread's last error; returns `code`. */
int pkv__fail(int code, const char* fmt, ...)
#if defined(__GNUC__) || defined(__clang__)
    __attribute__((format(printf, 2, 3)))
#endif
    ;

/* Clear this thread's last error. */
void pkv__clear_error(void);

/* Basic checks of a cache descriptor shared by every device call. */
int pkv__check_desc(const pkv_cache_desc* c);

/* Non-zero when the environment sets PKV_VALIDATE to a value other than "0"
 * (read on every call): the device calls then copy their index arrays to the
 * host, synchronously, and check them before launching anything. */
int pkv__validate_enabled(void);

/* Copy `bytes` from device (or pinned host) memory to host memory after the
 * work already queued on `stream` (a hipStream_t), synchronously; used by the
 * PKV_VALIDATE checks only.  PKV_EHIP on error. */
int pkv__copy_to_host(void* dst, const void* src, size_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_INTERNAL_H */
