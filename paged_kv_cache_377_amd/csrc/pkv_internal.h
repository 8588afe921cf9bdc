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

#ifdef __cplusplus
}
#endif

#endif /* PKV_INTERNAL_H */
